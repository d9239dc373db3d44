// FBI-linear backward through the straight-through estimator (FBI-LLM news
// rewrite, training paragraph: the STE carries gradients through the sign
// function, taken here as the identity since no clipping is stated). With
// y = alpha_j sum_i s_ij x_mi and the output gradient dY:
//   dX[m][i] = sum_j s_ij (alpha_j dY[m][j])      -- a product with S^T
//   dalpha_j = sum_m dY[m][j] z[m][j], z = x S     -- the forward at alpha = 1
//   dW[i][j] = alpha_j sum_m x[m][i] dY[m][j]      -- a dense product over tokens
//
// dX runs on the forward kernels: S^T is packed once (pack_transpose_kernel)
// in the forward's format, twice along its contraction axis, and the scaled
// gradient g = alpha * dY (fp32) enters as two 16-bit halves g_hi = bf16(g),
// g_lo = bf16(g - g_hi) laid side by side ([M][2N]): sum_j s_ij (g_hi + g_lo)
// carries g to about 16 significant bits, where a single bf16 copy of g would
// carry 8.
#include "bgb_device.hpp"
#include "bgb_internal.hpp"

namespace bgb {

// ---------------------------------------------------------- S^T, packed ----
// One wave per (32-row word t of S, 64 columns j0..j0+63): lane L holds word
// (t, j0 + L); the 32 ballots over bit b give, for row i = 32 t + b of S,
// the bits of columns j0..j0+63, i.e. words (j0 / 32, i) and (j0 / 32 + 1, i)
// of S^T, stored in both copies (rows j and N + j of the doubled matrix).
// Requires N % 32 == 0 (whole words per copy).
__global__ void __launch_bounds__(256)
pack_transpose_kernel(const uint32_t* __restrict__ P, int64_t K, int64_t N, uint32_t* __restrict__ PT) {
    const int lane = threadIdx.x & 63;
    const int64_t wid = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t nj = (N + 63) / 64, T = K / 32;
    if (wid >= T * nj) return;                          // uniform per wave
    const int64_t t = wid / nj, j0 = (wid % nj) * 64;
    const int64_t j = j0 + lane;
    const uint32_t w = j < N ? P[((t >> 2) * N + j) * 4 + (t & 3)] : 0u;
    uint64_t mine = 0;                                  // lane b < 32 keeps the ballot of bit b
#pragma unroll
    for (int b = 0; b < 32; ++b) {
        const uint64_t m = __ballot((w >> b) & 1u);
        mine = lane == b ? m : mine;
    }
    if (lane >= 32) return;
    const int64_t i = 32 * t + lane;                    // column of S^T
    const int64_t half = N / 32;                        // words per copy along the contraction axis
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t tw = j0 / 32 + h;                 // word of S^T in the first copy
        if (tw >= half) break;
        const uint32_t word = uint32_t(mine >> (32 * h));
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int64_t tt = tw + c * half;
            PT[((tt >> 2) * K + i) * 4 + (tt & 3)] = word;
        }
    }
}

// Zero words of the last 128-row tile past the doubled contraction axis
// (2N / 32 words when that is not a multiple of 4).
__global__ void __launch_bounds__(256)
pack_transpose_pad_kernel(int64_t K, int64_t T2, int64_t TQ2, uint32_t* __restrict__ PT) {
    const int64_t n = (4 * TQ2 - T2) * K;
    const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (e >= n) return;
    const int64_t tt = T2 + e / K, i = e % K;
    PT[((tt >> 2) * K + i) * 4 + (tt & 3)] = 0u;
}

hipError_t launch_pack_transpose(const uint32_t* P, int64_t K, int64_t N, uint32_t* PT, hipStream_t s) {
    const int64_t waves = (K / 32) * ((N + 63) / 64);
    pack_transpose_kernel<<<unsigned((waves + 3) / 4), 256, 0, s>>>(P, K, N, PT);
    const int64_t T2 = 2 * N / 32, TQ2 = tiles_per_col(2 * N);
    const int64_t pad = (4 * TQ2 - T2) * K;
    if (pad > 0) pack_transpose_pad_kernel<<<unsigned((pad + 255) / 256), 256, 0, s>>>(K, T2, TQ2, PT);
    return hipGetLastError();
}

// ------------------------------------------------------ g = alpha * dY -----
// g = fl32(dY alpha_j); row m of the output holds bf16(g) for j < N and
// bf16(g - bf16(g)) at N + j (g - bf16(g) is exact in fp32). A thread takes
// 8 consecutive columns (16-byte loads and stores; N % 8 == 0).
__global__ void __launch_bounds__(256)
split_scaled_grad_kernel(const uint16_t* __restrict__ dy, int dy_f16, int64_t M, int64_t N,
                         const void* __restrict__ alpha, int alpha_f16, uint16_t* __restrict__ g2) {
    const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t n8 = N / 8;
    if (e >= M * n8) return;
    const int64_t m = e / n8, j0 = (e % n8) * 8;
    const u32x4_t d = *reinterpret_cast<const u32x4_t*>(dy + m * N + j0);
    float a[8];
    if (alpha_f16) {
        const u32x4_t h = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(alpha) + j0);
#pragma unroll
        for (int k = 0; k < 8; ++k) a[k] = f16_to_f32(uint16_t(h[k >> 1] >> (16 * (k & 1))));
    } else {
        const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(alpha) + j0);
        const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(alpha) + j0 + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            a[k] = lo[k];
            a[4 + k] = hi[k];
        }
    }
    u32x4_t oh, ol;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint16_t b = uint16_t(d[k >> 1] >> (16 * (k & 1)));
        const float g = (dy_f16 ? f16_to_f32(b) : bf16_to_f32(b)) * a[k];
        const uint16_t h = f32_to_bf16_rne(g);
        const uint16_t l = f32_to_bf16_rne(g - bf16_to_f32(h));
        if (k & 1) {
            oh[k >> 1] |= uint32_t(h) << 16;
            ol[k >> 1] |= uint32_t(l) << 16;
        } else {
            oh[k >> 1] = h;
            ol[k >> 1] = l;
        }
    }
    *reinterpret_cast<u32x4_t*>(g2 + m * 2 * N + j0) = oh;
    *reinterpret_cast<u32x4_t*>(g2 + m * 2 * N + N + j0) = ol;
}

__global__ void __launch_bounds__(256) fill_ones_kernel(float* __restrict__ p, int64_t n) {
    const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (e < n) p[e] = 1.0f;
}

// ------------------------------------------------ dalpha = sum_m dY z ------
// Two passes, fixed order: a block takes 256 columns and a chunk of
// kDaChunk tokens; thread (c, q) sums tokens q, q + 4, ... of the chunk for
// columns 4c .. 4c + 3 in fp64 (the products of dY and z), the four q parts
// are added in order through LDS, and the chunk sums are added in chunk
// order by a second kernel.
constexpr int kDaChunk = 256;

__global__ void __launch_bounds__(256)
dalpha_part_kernel(const uint16_t* __restrict__ dy, int dy_f16, const float* __restrict__ z, int64_t M, int64_t N,
                   double* __restrict__ part) {
    __shared__ double red[4][64][4];
    const int c = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int64_t j = int64_t(blockIdx.x) * 256 + 4 * c, m0 = int64_t(blockIdx.y) * kDaChunk;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    if (j < N) {                                        // N % 4 == 0: 4 columns are all in or all out
        const int64_t m1 = m0 + kDaChunk < M ? m0 + kDaChunk : M;
        for (int64_t m = m0 + q; m < m1; m += 4) {
            const uint2 d = *reinterpret_cast<const uint2*>(dy + m * N + j);
            const f32x4_t zv = *reinterpret_cast<const f32x4_t*>(z + m * N + j);
            const uint32_t dw[2] = {d.x, d.y};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint16_t b = uint16_t(dw[k >> 1] >> (16 * (k & 1)));
                acc[k] += double(dy_f16 ? f16_to_f32(b) : bf16_to_f32(b)) * double(zv[k]);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) red[q][c][k] = acc[k];
    __syncthreads();
    if (q == 0 && j < N) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            part[int64_t(blockIdx.y) * N + j + k] = ((red[0][c][k] + red[1][c][k]) + red[2][c][k]) + red[3][c][k];
    }
}

__global__ void __launch_bounds__(256)
dalpha_sum_kernel(const double* __restrict__ part, int64_t chunks, int64_t N, float* __restrict__ dalpha) {
    const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (j >= N) return;
    double acc = 0.0;
    for (int64_t c = 0; c < chunks; ++c) acc += part[c * N + j];
    dalpha[j] = float(acc);
}

// ------------------------------------------- dW = alpha * (x^T dY) --------
// Dense 16-bit product over the tokens. A block computes a T x T tile of dW
// (T = 256: 8 waves, each 64 j x 128 i as 4 x 8 MFMA fragments) with A =
// dY^T (rows j) and B = x (columns i), so a lane's 4 outputs are 4
// consecutive j of one i (one 16-byte store). The tile size sets how often x
// and dY are re-read (by N / T and K / T blocks). Each
// chunk of 64 tokens is staged in LDS transposed (row = feature, the chunk's
// tokens contiguous), so that an operand is one 16-byte read: the first T
// threads load 8 tokens x 8 features of x, the other T the same of dY
// (16-byte loads, T / 8 threads per row piece), transpose the 8 x 8 block in
// registers (one v_perm per output dword) and store 8 rows of 16 bytes. Two
// LDS buffers: the next chunk is stored while the current one is multiplied
// and the one after it is loaded. Tokens past M and features past K or N
// read as zeros.
constexpr int kDwChunk = 64, kDwRow = kDwChunk + 8;   // LDS row: 64 tokens + 16 bytes
// The 8 token slots (16 bytes each) of a row are XOR-swizzled by bits 4..6 of
// the row: a store instruction writes rows 8 apart across its lanes (one
// feature of each lane's 8 x 8 block), which the 16-byte padding alone maps
// onto two 16-byte bank groups per 256 bytes; with the swizzle every 16
// consecutive lanes hit 16 distinct groups, and the reads (16 consecutive
// rows, one slot) stay distinct too.
BGB_DEV int dw_swz(int row) { return (row >> 4) & 7; }

// T: the square output tile (128 or 256), 2 T threads (T / 32 waves); wave w
// takes 64 j x 64 BI i (BI = T / 128): 4 x 4 BI MFMA fragments.
template <bool kF16, int T>
__global__ void __launch_bounds__(2 * T)
dw_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ dy, int64_t M, int64_t K, int64_t N,
          const void* __restrict__ alpha, int alpha_f16, float* __restrict__ dw) {
    constexpr int BI = T / 128;
    __shared__ __attribute__((aligned(16))) uint16_t xt[2][T * kDwRow];
    __shared__ __attribute__((aligned(16))) uint16_t gt[2][T * kDwRow];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
    const int64_t i0 = int64_t(blockIdx.x) * T, j0 = int64_t(blockIdx.y) * T;
    // waves: T / 64 columns of 64 j, 2 rows of 64 BI i
    const int wj = (wave % (T / 64)) * 64, wi = (wave / (T / 64)) * 64 * BI;

    // loader: half h (0: x, 1: dY), token rows 8 mb .. 8 mb + 7 of the chunk,
    // features 8 fb .. 8 fb + 7 of the tile (T / 8 threads per token row)
    const int h = tid / T, mb = (tid % T) / (T / 8), fb = tid % (T / 8);
    const uint16_t* src = h ? dy : x;
    const int64_t ld = h ? N : K;
    const int64_t f0 = (h ? j0 : i0) + 8 * fb;          // K, N multiples of 32: 8-feature pieces are whole
    const bool okf = f0 < ld;
    u32x4_t v[8];
    auto load = [&](int64_t m0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t m = m0 + 8 * mb + e;
            const bool ok = okf && m < M;
            const u32x4_t t = *reinterpret_cast<const u32x4_t*>(src + (ok ? m * ld + f0 : 0));
            v[e] = t & u32x4_t(0u - uint32_t(ok));
        }
    };
    auto store = [&](int buf) {
        uint16_t* const tile = h ? gt[buf] : xt[buf];
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            const uint32_t sel = (f & 1) ? 0x07060302u : 0x05040100u;
            u32x4_t o;
            o.x = __builtin_amdgcn_perm(v[1][f >> 1], v[0][f >> 1], sel);
            o.y = __builtin_amdgcn_perm(v[3][f >> 1], v[2][f >> 1], sel);
            o.z = __builtin_amdgcn_perm(v[5][f >> 1], v[4][f >> 1], sel);
            o.w = __builtin_amdgcn_perm(v[7][f >> 1], v[6][f >> 1], sel);
            const int row = 8 * fb + f;
            *reinterpret_cast<u32x4_t*>(tile + row * kDwRow + 8 * (mb ^ dw_swz(row))) = o;
        }
    };

    f32x4_t acc[4][4 * BI];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4 * BI; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // two LDS buffers: chunk c + 1 is stored into one while chunk c is
    // multiplied from the other, and chunk c + 2 is loaded meanwhile; one
    // barrier per chunk
    load(0);
    store(0);
    if (kDwChunk < M) load(kDwChunk);
    __syncthreads();
    int buf = 0;
    for (int64_t m0 = 0; m0 < M; m0 += kDwChunk, buf ^= 1) {
        if (m0 + kDwChunk < M) store(buf ^ 1);
        if (m0 + 2 * kDwChunk < M) load(m0 + 2 * kDwChunk);
        const uint16_t* const gb = gt[buf];
        const uint16_t* const xb = xt[buf];
#pragma unroll
        for (int ks = 0; ks < kDwChunk / 32; ++ks) {
            u32x4_t av[4], bv[4 * BI];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int row = wj + 16 * f + r;
                av[f] = *reinterpret_cast<const u32x4_t*>(gb + row * kDwRow + 8 * ((4 * ks + g) ^ dw_swz(row)));
            }
#pragma unroll
            for (int f = 0; f < 4 * BI; ++f) {
                const int row = wi + 16 * f + r;
                bv[f] = *reinterpret_cast<const u32x4_t*>(xb + row * kDwRow + 8 * ((4 * ks + g) ^ dw_swz(row)));
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4 * BI; ++b) {
                    if constexpr (kF16)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, av[a]),
                                                                           __builtin_bit_cast(f16x8_t, bv[b]),
                                                                           acc[a][b], 0, 0, 0);
                    else
                        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[a]),
                                                                            __builtin_bit_cast(bf16x8_t, bv[b]),
                                                                            acc[a][b], 0, 0, 0);
                }
        }
        __syncthreads();                                   // chunk c + 1 is in; chunk c's buffer is free
    }
    // lane (g, r) of fragment (a, b): j = j0 + wj + 16 a + 4 g + e, i = i0 + wi + 16 b + r
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int64_t jb = j0 + wj + 16 * a + 4 * g;
        if (jb >= N) continue;                             // N % 32 == 0: 4 columns are all in or all out
        float al[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            al[e] = alpha_f16 ? f16_to_f32(static_cast<const uint16_t*>(alpha)[jb + e])
                              : static_cast<const float*>(alpha)[jb + e];
#pragma unroll
        for (int b = 0; b < 4 * BI; ++b) {
            const int64_t i = i0 + wi + 16 * b + r;
            if (i >= K) continue;
            *reinterpret_cast<f32x4_t*>(dw + i * N + jb) =
                f32x4_t{al[0] * acc[a][b][0], al[1] * acc[a][b][1], al[2] * acc[a][b][2], al[3] * acc[a][b][3]};
        }
    }
}

hipError_t launch_fbi_backward_parts(const void* dy, int dy_f16, const void* x, int64_t M, int64_t K, int64_t N,
                                     const void* alpha, int alpha_f16, uint16_t* g2, float* ones, int64_t nones,
                                     float* dw, hipStream_t s) {
    if (g2) {
        const int64_t n = M * (N / 8);
        split_scaled_grad_kernel<<<unsigned((n + 255) / 256), 256, 0, s>>>(static_cast<const uint16_t*>(dy), dy_f16,
                                                                            M, N, alpha, alpha_f16, g2);
    }
    if (ones) fill_ones_kernel<<<unsigned((nones + 255) / 256), 256, 0, s>>>(ones, nones);
    if (dw) {
        constexpr int T = 256;                   // 8 waves, one block per CU (231 VGPRs; 128: 935 us, 256: 710 us)
        const dim3 grid(unsigned((K + T - 1) / T), unsigned((N + T - 1) / T));
        const uint16_t* xx = static_cast<const uint16_t*>(x);
        const uint16_t* gg = static_cast<const uint16_t*>(dy);
        if (dy_f16) dw_kernel<true, T><<<grid, 2 * T, 0, s>>>(xx, gg, M, K, N, alpha, alpha_f16, dw);
        else dw_kernel<false, T><<<grid, 2 * T, 0, s>>>(xx, gg, M, K, N, alpha, alpha_f16, dw);
    }
    return hipGetLastError();
}

hipError_t launch_dalpha(const void* dy, int dy_f16, const float* z, int64_t M, int64_t N, double* part,
                         float* dalpha, hipStream_t s) {
    const int64_t chunks = (M + kDaChunk - 1) / kDaChunk;
    dalpha_part_kernel<<<dim3(unsigned((N + 255) / 256), unsigned(chunks)), 256, 0, s>>>(
        static_cast<const uint16_t*>(dy), dy_f16, z, M, N, part);
    dalpha_sum_kernel<<<unsigned((N + 255) / 256), 256, 0, s>>>(part, chunks, N, dalpha);
    return hipGetLastError();
}

size_t dalpha_part_bytes(int64_t M, int64_t N) { return size_t((M + kDaChunk - 1) / kDaChunk) * size_t(N) * 8; }

}  // namespace bgb
