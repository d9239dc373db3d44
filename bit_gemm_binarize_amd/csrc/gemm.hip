// Prefill kernels (M > 16): a dense contraction, so it runs on the matrix
// cores. FBI-linear W1A16 (FBI-LLM news rewrite, FBI-linear paragraph) on
// bf16/f16 MFMA with fp32 accumulation; BitLinear W1A8 ("BitNet b1.58: 1bit
// LLM时代", section 一, eq. (7)) on int8 MFMA with int32 accumulation.
//
// Tiling: a block of 4 waves computes a 256-column x 128-token tile; wave w
// owns columns 64w..64w+63 (four 16-column MFMA fragments) for all 128
// tokens (eight 16-token fragments): 32 accumulators of 16x16. The K loop
// steps one 128-row column tile at a time. Activations are staged through
// LDS (double-buffered, rows padded by 16 bytes so the 16 lanes of a lane
// group hit distinct banks); the sign words go straight from global memory
// into registers -- lane group g of a fragment reads word g (rows 32g..32g+31
// of the tile) of its column -- and are decoded there into the MFMA A
// operand (rows of A = output columns). The C fragment then holds four
// consecutive output columns of one token per lane.
//
// Decoding, per MFMA:
// * W1A16, MFMA u = 0..3 of a 32-row word: dword e carries rows 4u+e (low
//   half) and 4u+e+16 (high half): ((~w << (15-4u-e)) & 0x80008000) | one,
//   i.e. +-1.0 with the sign bit taken from the weight bit. The activation
//   tile is stored in LDS with the two 16-row halves of each word
//   interleaved element by element so that the B operand matches.
// * W1A8, MFMA v = 0..1 of a word: dword d carries rows 4v+d+8e (byte e) as
//   0/1 bytes ((w >> (4v+d)) & 0x01010101); sum s q = 2 sum b q - sum q with
//   the row sums of the codes from the prologue. The prologue writes the
//   codes already in this order.
// Tiles are ranked XCD by XCD so that one XCD's L2 sees a contiguous run of
// tiles sharing activation rows.
#include "bgb_device.hpp"
#include "bgb_internal.hpp"

namespace bgb {

constexpr int kBM = 128;      // tokens per block tile
constexpr int kBJ = 256;      // output columns per block tile
constexpr int kRow16 = 272;   // LDS bytes per token row, 16-bit tile (256 + 16 pad)
constexpr int kRow8 = 144;    // LDS bytes per token row, int8 tile (128 + 16 pad)

template <bool kF16>
BGB_DEV f32x4_t mfma16g(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
    if constexpr (kF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

BGB_DEV void store_y16(void* y, int y_dtype, int64_t i, float v) {
    if (y_dtype == kDtF32) static_cast<float*>(y)[i] = v;
    else if (y_dtype == kDtBF16) static_cast<uint16_t*>(y)[i] = f32_to_bf16_rne(v);
    else static_cast<uint16_t*>(y)[i] = f32_to_f16_rne(v);
}

BGB_DEV float alpha_at(const void* alpha, int alpha_f16, int64_t j) {
    return alpha_f16 ? f16_to_f32(static_cast<const uint16_t*>(alpha)[j]) : static_cast<const float*>(alpha)[j];
}

template <bool kF16>
__global__ void __launch_bounds__(256, 2)
gemm_w1a16_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t N, int64_t TQ,
                  const uint32_t* __restrict__ P, const void* __restrict__ alpha, int alpha_f16,
                  void* __restrict__ y, int y_dtype, int ntj, int ntiles) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][kBM * kRow16];
    const int tile = xcd_tile(blockIdx.x, ntiles);
    if (tile >= ntiles) return;
    const int64_t m0 = int64_t(tile / ntj) * kBM, j0 = int64_t(tile % ntj) * kBJ;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
    constexpr uint32_t kOne = kF16 ? 0x3C003C00u : 0x3F803F80u;

    // staging: each thread moves 4 (row, word, half-pair) tasks per tile:
    // 2 x 16 bytes in (rows k..k+7 and k+16..k+23 of one word), 32 bytes out.
    u32x4_t stg[4][2];
    auto gload = [&](int64_t tq) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int task = tid + 256 * i;
            const int row = task >> 3, gw = (task >> 1) & 3, hp = task & 1;
            const int64_t m = m0 + row;
            const int64_t k = tq * 128 + 32 * gw + 8 * hp;
            u32x4_t lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
            if (m < M && k < K) {
                const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + m * K + k);
                lo = src[0];
                hi = src[2];
            }
            stg[i][0] = lo;
            stg[i][1] = hi;
        }
    };
    auto lwrite = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int task = tid + 256 * i;
            const int row = task >> 3, gw = (task >> 1) & 3, hp = task & 1;
            u32x4_t* dst = reinterpret_cast<u32x4_t*>(&lds[buf][row * kRow16 + gw * 64 + hp * 32]);
            const u32x4_t lo = stg[i][0], hi = stg[i][1];
            u32x4_t o0, o1;
            o0.x = __builtin_amdgcn_perm(hi.x, lo.x, 0x05040100u);
            o0.y = __builtin_amdgcn_perm(hi.x, lo.x, 0x07060302u);
            o0.z = __builtin_amdgcn_perm(hi.y, lo.y, 0x05040100u);
            o0.w = __builtin_amdgcn_perm(hi.y, lo.y, 0x07060302u);
            o1.x = __builtin_amdgcn_perm(hi.z, lo.z, 0x05040100u);
            o1.y = __builtin_amdgcn_perm(hi.z, lo.z, 0x07060302u);
            o1.z = __builtin_amdgcn_perm(hi.w, lo.w, 0x05040100u);
            o1.w = __builtin_amdgcn_perm(hi.w, lo.w, 0x07060302u);
            dst[0] = o0;
            dst[1] = o1;
        }
    };
    uint32_t wcur[4], wnxt[4];
    auto wload = [&](int64_t tq, uint32_t* wd) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int64_t jf = j0 + 64 * wave + 16 * f + r;
            wd[f] = jf < N ? P[(tq * N + jf) * 4 + g] : 0u;
        }
    };

    f32x4_t acc[4][8];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[f][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    gload(0);
    wload(0, wcur);
    lwrite(0);
    __syncthreads();
    for (int64_t tq = 0; tq < TQ; ++tq) {
        const int buf = int(tq & 1);
        const bool more = tq + 1 < TQ;
        if (more) {
            gload(tq + 1);
            wload(tq + 1, wnxt);
        }
        const uint8_t* lb = lds[buf];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            u32x4_t b[8];
#pragma unroll
            for (int n = 0; n < 8; ++n)
                b[n] = *reinterpret_cast<const u32x4_t*>(lb + (16 * n + r) * kRow16 + g * 64 + u * 16);
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const uint32_t nw = ~wcur[f];
                u32x4_t a;
                a.x = ((nw << (15 - 4 * u)) & 0x80008000u) | kOne;
                a.y = ((nw << (14 - 4 * u)) & 0x80008000u) | kOne;
                a.z = ((nw << (13 - 4 * u)) & 0x80008000u) | kOne;
                a.w = ((nw << (12 - 4 * u)) & 0x80008000u) | kOne;
#pragma unroll
                for (int n = 0; n < 8; ++n) acc[f][n] = mfma16g<kF16>(a, b[n], acc[f][n]);
            }
        }
        if (more) {
            lwrite(buf ^ 1);
#pragma unroll
            for (int f = 0; f < 4; ++f) wcur[f] = wnxt[f];
        }
        __syncthreads();
    }

#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int64_t jb = j0 + 64 * wave + 16 * f + 4 * g;
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = jb + i < N ? alpha_at(alpha, alpha_f16, jb + i) : 0.0f;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const int64_t m = m0 + 16 * n + r;
            if (m >= M) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (jb + i < N) store_y16(y, y_dtype, m * N + jb + i, al[i] * acc[f][n][i]);
        }
    }
}

hipError_t launch_w1a16_gemm(const void* x, int x_f16, int64_t M, int64_t K, int64_t N, const uint32_t* P,
                             const void* alpha, int alpha_f16, void* y, int y_dtype, hipStream_t s) {
    const int ntj = int((N + kBJ - 1) / kBJ), ntm = int((M + kBM - 1) / kBM);
    const int ntiles = ntj * ntm;
    const unsigned grid = unsigned(xcd_grid(ntiles));
    const uint16_t* xx = static_cast<const uint16_t*>(x);
    if (x_f16)
        gemm_w1a16_kernel<true><<<grid, 256, 0, s>>>(xx, M, K, N, tiles_per_col(K), P, alpha, alpha_f16, y, y_dtype,
                                                      ntj, ntiles);
    else
        gemm_w1a16_kernel<false><<<grid, 256, 0, s>>>(xx, M, K, N, tiles_per_col(K), P, alpha, alpha_f16, y,
                                                       y_dtype, ntj, ntiles);
    return hipGetLastError();
}

// ------------------------------------------------------------------- W1A8 ----
__global__ void __launch_bounds__(256, 2)
gemm_w1a8_kernel(const int8_t* __restrict__ q, const int32_t* __restrict__ rowsum, const float* __restrict__ gamma,
                 const float* __restrict__ beta, float qb, int64_t M, int64_t N, int64_t TQ,
                 const uint32_t* __restrict__ P, float* __restrict__ y, int32_t* __restrict__ acc_opt, int ntj,
                 int ntiles) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][kBM * kRow8];
    const int tile = xcd_tile(blockIdx.x, ntiles);
    if (tile >= ntiles) return;
    const int64_t m0 = int64_t(tile / ntj) * kBM, j0 = int64_t(tile % ntj) * kBJ;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
    const int64_t Kp = TQ * 128;

    u32x4_t stg[4];
    auto gload = [&](int64_t tq) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int task = tid + 256 * i;
            const int row = task >> 3, c = task & 7;
            const int64_t m = m0 + row;
            stg[i] = m < M ? *reinterpret_cast<const u32x4_t*>(q + m * Kp + tq * 128 + 16 * c)
                           : u32x4_t{0u, 0u, 0u, 0u};
        }
    };
    auto lwrite = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int task = tid + 256 * i;
            const int row = task >> 3, c = task & 7;
            *reinterpret_cast<u32x4_t*>(&lds[buf][row * kRow8 + 16 * c]) = stg[i];
        }
    };
    uint32_t wcur[4], wnxt[4];
    auto wload = [&](int64_t tq, uint32_t* wd) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int64_t jf = j0 + 64 * wave + 16 * f + r;
            wd[f] = jf < N ? P[(tq * N + jf) * 4 + g] : 0u;
        }
    };

    i32x4_t acc[4][8];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[f][n] = i32x4_t{0, 0, 0, 0};

    gload(0);
    wload(0, wcur);
    lwrite(0);
    __syncthreads();
    for (int64_t tq = 0; tq < TQ; ++tq) {
        const int buf = int(tq & 1);
        const bool more = tq + 1 < TQ;
        if (more) {
            gload(tq + 1);
            wload(tq + 1, wnxt);
        }
        const uint8_t* lb = lds[buf];
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            i32x4_t b[8];
#pragma unroll
            for (int n = 0; n < 8; ++n)
                b[n] = *reinterpret_cast<const i32x4_t*>(lb + (16 * n + r) * kRow8 + g * 32 + v * 16);
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const uint32_t w = wcur[f];
                i32x4_t a;
                a.x = int((w >> (4 * v + 0)) & 0x01010101u);
                a.y = int((w >> (4 * v + 1)) & 0x01010101u);
                a.z = int((w >> (4 * v + 2)) & 0x01010101u);
                a.w = int((w >> (4 * v + 3)) & 0x01010101u);
#pragma unroll
                for (int n = 0; n < 8; ++n)
                    acc[f][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[n], acc[f][n], 0, 0, 0);
            }
        }
        if (more) {
            lwrite(buf ^ 1);
#pragma unroll
            for (int f = 0; f < 4; ++f) wcur[f] = wnxt[f];
        }
        __syncthreads();
    }

    const float scale = (beta[0] * gamma[0]) / qb;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int64_t jb = j0 + 64 * wave + 16 * f + 4 * g;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const int64_t m = m0 + 16 * n + r;
            if (m >= M) continue;
            const int32_t rs = rowsum[m];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (jb + i >= N) continue;
                const int32_t a = 2 * acc[f][n][i] - rs;
                y[m * N + jb + i] = float(a) * scale;
                if (acc_opt) acc_opt[m * N + jb + i] = a;
            }
        }
    }
}

hipError_t launch_w1a8_gemm(const int8_t* q, const int32_t* rowsum, const float* gamma, const float* beta, float qb,
                            int64_t M, int64_t K, int64_t N, const uint32_t* P, float* y, int32_t* acc_opt,
                            hipStream_t s) {
    const int ntj = int((N + kBJ - 1) / kBJ), ntm = int((M + kBM - 1) / kBM);
    const int ntiles = ntj * ntm;
    gemm_w1a8_kernel<<<unsigned(xcd_grid(ntiles)), 256, 0, s>>>(q, rowsum, gamma, beta, qb, M, N, tiles_per_col(K),
                                                                  P, y, acc_opt, ntj, ntiles);
    return hipGetLastError();
}

}  // namespace bgb
