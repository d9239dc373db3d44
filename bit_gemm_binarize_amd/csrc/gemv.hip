// Decode kernels (M <= 16): stream the packed signs once from HBM and run the
// contraction on the matrix cores with the batch padded to 16 tokens.
//
// FBI-linear W1A16 (FBI-LLM news rewrite, FBI-linear paragraph):
//   y[m][j] = alpha_j * sum_k s_kj x[m][k]
// BitLinear W1A8 ("BitNet b1.58: 1bit LLM时代", section 一, eq. (7)):
//   acc[m][j] = sum_k s_kj q[m][k];  y = acc * beta * gamma / Q_b
//
// Work split: a block of 4 waves owns 16 output columns. Each wave takes
// every 4th "step" of 4 column tiles (512 rows); in a step lane group g
// (lanes 16g..16g+15) loads the 16-byte tile (4 words, 128 rows) of column
// j0 + (lane % 16) in tile 4*step + g, so one load instruction moves 1 KB.
// The MFMA A operand is built from these words (rows of A = columns j), the
// B operand is the activation slice of token (lane % 16); the 4 waves' partial
// sums are added in a fixed order through LDS.
//
// Sign decoding, written so that the only per-weight work is one AND (W1A8)
// or one AND-OR (W1A16) per pair/quad of weights:
// * W1A8: with b = 1 for +1, sum_k s q = 2 sum_k b q - sum_k q. The int8 MFMA
//   for shift s takes bytes (word & (0x01010101 << s)) -- the value 2^s b, or
//   -128 b for s = 7 -- from the 4 words of the tile, so it accumulates
//   2^s sum b q exactly; the 8 accumulators are shifted back and added.
// * W1A16: a 16-bit float whose exponent field is set and one low field bit
//   b is free encodes a + c b. MFMA u (0..15) takes bit u and bit u + 16 of
//   each word, moved by a per-u constant shift into field bit p = P0 + u % 4
//   (one shift per word for four MFMAs): p = P0..P0+2 are mantissa bits over a
//   base of 1.0 (a = 1, c = 1/8, 1/4, 1/2), p = P0+3 is the exponent's lowest
//   bit over a base of 0.5 (a = 1/2, c = 1/2). MFMAs of one type T = u % 4 share
//   an accumulator acc_T = a_T X_T + c_T sum_{k in T} b x, with X_T the sum of x
//   over the rows of type T (rows k with k % 4 == T), so
//   sum_k b x = sum_T (acc_T - a_T X_T) / c_T, exact scalings by powers of two.
#include "bgb_device.hpp"
#include "bgb_internal.hpp"

namespace bgb {

// ---------------------------------------------------------------- W1A16 prep --
// xp[m][128 tq + 8u + 2d + h] = x[m][32 (4 tq + d) + u + 16 h]  (0 beyond K),
// xsum[m][T] = sum of x[m][k] over k % 4 == T (fp32, fixed order).
__global__ void __launch_bounds__(256)
w1a16_prep_kernel(const uint16_t* __restrict__ x, int64_t K, int64_t Kp, int is_f16,
                  uint16_t* __restrict__ xp, float* __restrict__ xsum) {
    __shared__ double dscr[4];
    const int64_t m = blockIdx.x;
    const uint16_t* xr = x + m * K;
    uint16_t* out = xp + m * Kp;
    for (int64_t p = threadIdx.x; p < Kp; p += 256) {
        const int64_t tq = p / 128;
        const int r = int(p % 128);
        const int u = r >> 3, d = (r >> 1) & 3, h = r & 1;
        const int64_t k = 32 * (4 * tq + d) + u + 16 * h;
        out[p] = k < K ? xr[k] : uint16_t(0);
    }
    for (int T = 0; T < 4; ++T) {
        double s = 0.0;
        for (int64_t k = 4 * int64_t(threadIdx.x) + T; k < K; k += 4 * 256)
            s += double(is_f16 ? f16_to_f32(xr[k]) : bf16_to_f32(xr[k]));
        s = block_sum<256>(s, dscr);
        if (threadIdx.x == 0) xsum[4 * m + T] = float(s);
    }
}

hipError_t launch_w1a16_prep(const void* x, int is_f16, int64_t M, int64_t K, uint16_t* xp, float* xsum,
                                hipStream_t s) {
    w1a16_prep_kernel<<<unsigned(M), 256, 0, s>>>(static_cast<const uint16_t*>(x), K, padded_k(K), is_f16, xp,
                                                  xsum);
    return hipGetLastError();
}

// Field-bit constants per 16-bit format: P0 = first field bit used, the
// 1.0 and 0.5 bases (replicated in both halves of a dword).
template <bool kF16> struct Fmt16;
template <> struct Fmt16<false> {   // bf16: 7 mantissa bits, exponent LSB = bit 7
    static constexpr int P0 = 4;
    static constexpr uint32_t kOne = 0x3F803F80u, kHalf = 0x3F003F00u;
};
template <> struct Fmt16<true> {    // f16: 10 mantissa bits, exponent LSB = bit 10
    static constexpr int P0 = 7;
    static constexpr uint32_t kOne = 0x3C003C00u, kHalf = 0x38003800u;
};

template <bool kF16>
BGB_DEV f32x4_t mfma16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
    if constexpr (kF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int kShift>
BGB_DEV uint32_t shift_word(uint32_t w) {
    if constexpr (kShift >= 0) return w << kShift;
    else return w >> (-kShift);
}

// One MFMA u of a step: A dwords from the four words' bit pair (u, u+16).
template <bool kF16, int U>
BGB_DEV void w1a16_mfma_u(const u32x4_t& w, const u32x4_t& b, f32x4_t* acc) {
    using F = Fmt16<kF16>;
    constexpr int T = U % 4;
    constexpr int p = F::P0 + T;
    constexpr int sh = p - U;
    constexpr uint32_t mask = 0x00010001u << p;
    constexpr uint32_t base = (T == 3) ? F::kHalf : F::kOne;
    u32x4_t a;
    a.x = (shift_word<sh>(w.x) & mask) | base;
    a.y = (shift_word<sh>(w.y) & mask) | base;
    a.z = (shift_word<sh>(w.z) & mask) | base;
    a.w = (shift_word<sh>(w.w) & mask) | base;
    acc[T] = mfma16<kF16>(a, b, acc[T]);
}

BGB_DEV void store_y(void* y, int y_dtype, int64_t i, float v) {
    if (y_dtype == kDtF32) static_cast<float*>(y)[i] = v;
    else if (y_dtype == kDtBF16) static_cast<uint16_t*>(y)[i] = f32_to_bf16_rne(v);
    else static_cast<uint16_t*>(y)[i] = f32_to_f16_rne(v);
}

BGB_DEV float load_alpha(const void* alpha, int alpha_f16, int64_t j) {
    return alpha_f16 ? f16_to_f32(static_cast<const uint16_t*>(alpha)[j]) : static_cast<const float*>(alpha)[j];
}

template <bool kF16>
__global__ void __launch_bounds__(256)
gemv_w1a16_kernel(const uint16_t* __restrict__ xp, const float* __restrict__ xsum, int M, int64_t N, int64_t TQ,
                  const uint32_t* __restrict__ P, const void* __restrict__ alpha, int alpha_f16,
                  void* __restrict__ y, int y_dtype) {
    __shared__ f32x4_t red[4][4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int64_t j0 = int64_t(blockIdx.x) * 16;
    const int64_t j = j0 + r;
    const int64_t Kp = TQ * 128;
    const int64_t steps = (TQ + 3) / 4;
    f32x4_t acc[4];
#pragma unroll
    for (int T = 0; T < 4; ++T) acc[T] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int64_t st = wave; st < steps; st += 4) {
        const int64_t tq = st * 4 + g;
        u32x4_t w = {0u, 0u, 0u, 0u};
        if (tq < TQ && j < N) w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(P + (tq * N + j) * 4));
        const bool bval = r < M && tq < TQ;
        const u32x4_t* xb = reinterpret_cast<const u32x4_t*>(xp + int64_t(r) * Kp + tq * 128);
        u32x4_t b[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) b[u] = bval ? xb[u] : u32x4_t{0u, 0u, 0u, 0u};
        w1a16_mfma_u<kF16, 0>(w, b[0], acc);   w1a16_mfma_u<kF16, 1>(w, b[1], acc);
        w1a16_mfma_u<kF16, 2>(w, b[2], acc);   w1a16_mfma_u<kF16, 3>(w, b[3], acc);
        w1a16_mfma_u<kF16, 4>(w, b[4], acc);   w1a16_mfma_u<kF16, 5>(w, b[5], acc);
        w1a16_mfma_u<kF16, 6>(w, b[6], acc);   w1a16_mfma_u<kF16, 7>(w, b[7], acc);
        w1a16_mfma_u<kF16, 8>(w, b[8], acc);   w1a16_mfma_u<kF16, 9>(w, b[9], acc);
        w1a16_mfma_u<kF16, 10>(w, b[10], acc); w1a16_mfma_u<kF16, 11>(w, b[11], acc);
        w1a16_mfma_u<kF16, 12>(w, b[12], acc); w1a16_mfma_u<kF16, 13>(w, b[13], acc);
        w1a16_mfma_u<kF16, 14>(w, b[14], acc); w1a16_mfma_u<kF16, 15>(w, b[15], acc);
    }
#pragma unroll
    for (int T = 0; T < 4; ++T) red[wave][T][lane] = acc[T];
    __syncthreads();
    if (wave != 0) return;
    f32x4_t tot[4];
#pragma unroll
    for (int T = 0; T < 4; ++T) tot[T] = ((red[0][T][lane] + red[1][T][lane]) + red[2][T][lane]) + red[3][T][lane];
    const int mm = r;                          // C column = token
    if (mm >= M) return;
    const float X0 = xsum[4 * mm], X1 = xsum[4 * mm + 1], X2 = xsum[4 * mm + 2], X3 = xsum[4 * mm + 3];
    const float xall = ((X0 + X1) + X2) + X3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t col = j0 + 4 * g + i;    // C row = column
        if (col >= N) continue;
        const float sb = ((8.0f * (tot[0][i] - X0) + 4.0f * (tot[1][i] - X1)) + 2.0f * (tot[2][i] - X2)) +
                         2.0f * (tot[3][i] - 0.5f * X3);
        const float s = 2.0f * sb - xall;
        store_y(y, y_dtype, int64_t(mm) * N + col, load_alpha(alpha, alpha_f16, col) * s);
    }
}

hipError_t launch_w1a16_gemv(const uint16_t* xp, const float* xsum, int x_f16, int64_t M, int64_t K, int64_t N,
                             const uint32_t* P, const void* alpha, int alpha_f16, void* y, int y_dtype,
                             hipStream_t s) {
    const unsigned grid = unsigned((N + 15) / 16);
    const int64_t TQ = tiles_per_col(K);
    if (x_f16)
        gemv_w1a16_kernel<true><<<grid, 256, 0, s>>>(xp, xsum, int(M), N, TQ, P, alpha, alpha_f16, y, y_dtype);
    else
        gemv_w1a16_kernel<false><<<grid, 256, 0, s>>>(xp, xsum, int(M), N, TQ, P, alpha, alpha_f16, y, y_dtype);
    return hipGetLastError();
}

// ------------------------------------------------------------------- W1A8 ----
template <int S>
BGB_DEV void w1a8_mfma_s(const u32x4_t& w, const i32x4_t& b, i32x4_t* acc) {
    constexpr uint32_t mask = 0x01010101u << S;
    const i32x4_t a = {int(w.x & mask), int(w.y & mask), int(w.z & mask), int(w.w & mask)};
    acc[S] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[S], 0, 0, 0);
}

__global__ void __launch_bounds__(256)
gemv_w1a8_kernel(const int8_t* __restrict__ q, const int32_t* __restrict__ rowsum, const float* __restrict__ gamma,
                 const float* __restrict__ beta, float qb, int M, int64_t N, int64_t TQ,
                 const uint32_t* __restrict__ P, float* __restrict__ y, int32_t* __restrict__ acc_opt) {
    __shared__ i32x4_t red[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int64_t j0 = int64_t(blockIdx.x) * 16;
    const int64_t j = j0 + r;
    const int64_t Kp = TQ * 128;
    const int64_t steps = (TQ + 3) / 4;
    i32x4_t acc[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[s] = i32x4_t{0, 0, 0, 0};
    for (int64_t st = wave; st < steps; st += 4) {
        const int64_t tq = st * 4 + g;
        u32x4_t w = {0u, 0u, 0u, 0u};
        if (tq < TQ && j < N) w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(P + (tq * N + j) * 4));
        const bool bval = r < M && tq < TQ;
        const i32x4_t* qb4 = reinterpret_cast<const i32x4_t*>(q + int64_t(r) * Kp + tq * 128);
        i32x4_t b[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) b[s] = bval ? qb4[s] : i32x4_t{0, 0, 0, 0};
        w1a8_mfma_s<0>(w, b[0], acc); w1a8_mfma_s<1>(w, b[1], acc);
        w1a8_mfma_s<2>(w, b[2], acc); w1a8_mfma_s<3>(w, b[3], acc);
        w1a8_mfma_s<4>(w, b[4], acc); w1a8_mfma_s<5>(w, b[5], acc);
        w1a8_mfma_s<6>(w, b[6], acc); w1a8_mfma_s<7>(w, b[7], acc);
    }
    // sum_k b q = sum_{s<7} acc_s / 2^s - acc_7 / 128 (each division exact)
    i32x4_t tot;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int t = 0;
#pragma unroll
        for (int s = 0; s < 7; ++s) t += acc[s][i] >> s;
        tot[i] = t - (acc[7][i] >> 7);
    }
    red[wave][lane] = tot;
    __syncthreads();
    if (wave != 0) return;
    const i32x4_t sum = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
    const int mm = r;
    if (mm >= M) return;
    const float scale = (beta[0] * gamma[0]) / qb;
    const int32_t rs = rowsum[mm];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t col = j0 + 4 * g + i;
        if (col >= N) continue;
        const int32_t a = 2 * sum[i] - rs;
        y[int64_t(mm) * N + col] = float(a) * scale;
        if (acc_opt) acc_opt[int64_t(mm) * N + col] = a;
    }
}

hipError_t launch_w1a8_gemv(const int8_t* q, const int32_t* rowsum, const float* gamma, const float* beta, float qb,
                            int64_t M, int64_t K, int64_t N, const uint32_t* P, float* y, int32_t* acc_opt,
                            hipStream_t s) {
    const unsigned grid = unsigned((N + 15) / 16);
    gemv_w1a8_kernel<<<grid, 256, 0, s>>>(q, rowsum, gamma, beta, qb, int(M), N, tiles_per_col(K), P, y, acc_opt);
    return hipGetLastError();
}

}  // namespace bgb
