// BitLinear prologue: per-token LayerNorm, tensor-wide absmax, b-bit codes.
//
// "BitNet b1.58: 1bit LLM时代" blog, section 一 (BitNet): eq. (8) LayerNorm
// (x - E x) / sqrt(Var x + eps); eq. (4)-(5) Quant(x) = Clip(x Q_b / gamma,
// -Q_b + eps, Q_b - eps) with gamma = ||x||_inf over the input matrix.
//
// Numerics (fixed so that codes are reproducible and identical to the
// reference): E x and Var x (biased, two passes) in fp64; mu32 = fl32(E x),
// rstd32 = fl32(1 / sqrt(Var x + eps)); h = fl32(fl32(x - mu32) * rstd32);
// gamma = max |h|; v = fl32(h Q_b / gamma) (h Q_b exact, one rounding);
// clip to +-lim with lim = fl32(Q_b - q_eps); truncate toward zero.
//
// The codes are written in the order the product kernels read them (one
// 128-row tile at a time, zero-padded to whole tiles):
//   layout 0 (decode kernel): dword (4s + d) of a tile holds rows 32d + s + 8e
//   layout 1 (GEMM kernel):   dword (8d + w) of a tile holds rows 32d + w + 8e
// for byte e = 0..3. The row sums of the codes are written too.
#include "bgb_device.hpp"
#include "bgb_internal.hpp"

namespace bgb {

template <typename XT> BGB_DEV float load_x(const XT* p, int64_t i);
template <> BGB_DEV float load_x<float>(const float* p, int64_t i) { return p[i]; }
template <> BGB_DEV float load_x<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

BGB_DEV float ln_apply(float x, float mu32, float rs32) { return (x - mu32) * rs32; }

BGB_DEV int quant_code(float h, float qb, float gamma, float lim) {
    if (gamma == 0.0f) return 0;
    float v = (h * qb) / gamma;
    v = fminf(fmaxf(v, -lim), lim);
    return int(v);   // truncation toward zero
}

// First row (within a 128-row tile) of the four codes packed in dword `dw`.
BGB_DEV int code_base(int layout, int dw) {
    return layout == 0 ? 32 * (dw & 3) + (dw >> 2) : 32 * (dw >> 3) + (dw & 7);
}

// mu32, rstd32 of one row, computed by a block of NT threads.
template <int NT, typename XT>
BGB_DEV void row_stats(const XT* xr, int64_t K, double eps, double* dscr, float& mu32, float& rs32) {
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < K; i += NT) s += double(load_x(xr, i));
    s = block_sum<NT>(s, dscr);
    const double mu = s / double(K);
    double v = 0.0;
    for (int64_t i = threadIdx.x; i < K; i += NT) {
        const double d = double(load_x(xr, i)) - mu;
        v += d * d;
    }
    v = block_sum<NT>(v, dscr);
    mu32 = float(mu);
    rs32 = float(1.0 / sqrt(v / double(K) + eps));
}

// Quantize one row with a block of NT threads; returns the row's code sum.
template <int NT, typename XT>
BGB_DEV int quant_row(const XT* xr, int64_t K, int64_t Kp, float mu32, float rs32, float qb, float gamma,
                      float lim, int layout, uint32_t* qrow, int8_t* natrow, int* iscr) {
    int sum = 0;
    for (int64_t dwi = threadIdx.x; dwi < Kp / 4; dwi += NT) {
        const int64_t k0 = (dwi / 32) * 128 + code_base(layout, int(dwi % 32));
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t k = k0 + 8 * e;
            int c = 0;
            if (k < K) {
                c = quant_code(ln_apply(load_x(xr, k), mu32, rs32), qb, gamma, lim);
                if (natrow) natrow[k] = int8_t(c);
            }
            sum += c;
            packed |= uint32_t(uint8_t(int8_t(c))) << (8 * e);
        }
        qrow[dwi] = packed;
    }
    return block_sum_i<NT>(sum, iscr);
}

// Small M (decode): the whole prologue in one block.
template <typename XT>
__global__ void __launch_bounds__(1024)
lnq_small_kernel(const XT* __restrict__ x, int M, int64_t K, int64_t Kp, double eps, float qb, float lim,
                 int layout, int8_t* __restrict__ q, int32_t* __restrict__ rowsum, float* __restrict__ stats,
                 float* __restrict__ gamma_ws, int8_t* __restrict__ xq_opt, float* __restrict__ gamma_opt) {
    __shared__ double dscr[16];
    __shared__ float fscr[16];
    __shared__ int iscr[16];
    __shared__ float s_mu[kSmallPrologueM], s_rs[kSmallPrologueM];
    float gmax = 0.0f;
    for (int m = 0; m < M; ++m) {
        const XT* xr = x + int64_t(m) * K;
        float mu32, rs32;
        row_stats<1024>(xr, K, eps, dscr, mu32, rs32);
        float lm = 0.0f;
        for (int64_t i = threadIdx.x; i < K; i += 1024) lm = fmaxf(lm, fabsf(ln_apply(load_x(xr, i), mu32, rs32)));
        lm = block_max<1024>(lm, fscr);
        if (threadIdx.x == 0) {
            s_mu[m] = mu32;
            s_rs[m] = rs32;
            stats[3 * m] = mu32;
            stats[3 * m + 1] = rs32;
            stats[3 * m + 2] = lm;
        }
        gmax = fmaxf(gmax, lm);
    }
    __syncthreads();
    const float gamma = gmax;
    if (threadIdx.x == 0) {
        gamma_ws[0] = gamma;
        if (gamma_opt) gamma_opt[0] = gamma;
    }
    for (int m = 0; m < M; ++m) {
        const int s = quant_row<1024>(x + int64_t(m) * K, K, Kp, s_mu[m], s_rs[m], qb, gamma, lim, layout,
                                      reinterpret_cast<uint32_t*>(q + int64_t(m) * Kp),
                                      xq_opt ? xq_opt + int64_t(m) * K : nullptr, iscr);
        if (threadIdx.x == 0) rowsum[m] = s;
    }
}

// Large M, pass 1: one block per row -> mu32, rstd32, max |h|.
template <typename XT>
__global__ void __launch_bounds__(256)
lnq_stats_kernel(const XT* __restrict__ x, int64_t K, double eps, float* __restrict__ stats) {
    __shared__ double dscr[4];
    __shared__ float fscr[4];
    const int64_t m = blockIdx.x;
    const XT* xr = x + m * K;
    float mu32, rs32;
    row_stats<256>(xr, K, eps, dscr, mu32, rs32);
    float lm = 0.0f;
    for (int64_t i = threadIdx.x; i < K; i += 256) lm = fmaxf(lm, fabsf(ln_apply(load_x(xr, i), mu32, rs32)));
    lm = block_max<256>(lm, fscr);
    if (threadIdx.x == 0) {
        stats[3 * m] = mu32;
        stats[3 * m + 1] = rs32;
        stats[3 * m + 2] = lm;
    }
}

// Large M, pass 2: gamma = max over the row maxima (every block computes the
// same exact maximum), then one block per row quantizes.
template <typename XT>
__global__ void __launch_bounds__(256)
lnq_quant_kernel(const XT* __restrict__ x, int64_t M, int64_t K, int64_t Kp, float qb, float lim, int layout,
                 const float* __restrict__ stats, int8_t* __restrict__ q, int32_t* __restrict__ rowsum,
                 float* __restrict__ gamma_ws, int8_t* __restrict__ xq_opt, float* __restrict__ gamma_opt) {
    __shared__ float fscr[4];
    __shared__ int iscr[4];
    float g = 0.0f;
    for (int64_t i = threadIdx.x; i < M; i += 256) g = fmaxf(g, stats[3 * i + 2]);
    const float gamma = block_max<256>(g, fscr);
    const int64_t m = blockIdx.x;
    if (m == 0 && threadIdx.x == 0) {
        gamma_ws[0] = gamma;
        if (gamma_opt) gamma_opt[0] = gamma;
    }
    const int s = quant_row<256>(x + m * K, K, Kp, stats[3 * m], stats[3 * m + 1], qb, gamma, lim, layout,
                                 reinterpret_cast<uint32_t*>(q + m * Kp), xq_opt ? xq_opt + m * K : nullptr, iscr);
    if (threadIdx.x == 0) rowsum[m] = s;
}

template <typename XT>
static void launch_lnq_t(const XT* x, int64_t M, int64_t K, double eps, float qb, float lim, int layout,
                         int8_t* q, int32_t* rowsum, float* stats, float* gamma_ws, int8_t* xq_opt,
                         float* gamma_opt, hipStream_t s) {
    const int64_t Kp = padded_k(K);
    if (M <= kSmallPrologueM) {
        lnq_small_kernel<XT><<<1, 1024, 0, s>>>(x, int(M), K, Kp, eps, qb, lim, layout, q, rowsum, stats,
                                                 gamma_ws, xq_opt, gamma_opt);
    } else {
        lnq_stats_kernel<XT><<<unsigned(M), 256, 0, s>>>(x, K, eps, stats);
        lnq_quant_kernel<XT><<<unsigned(M), 256, 0, s>>>(x, M, K, Kp, qb, lim, layout, stats, q, rowsum,
                                                          gamma_ws, xq_opt, gamma_opt);
    }
}

hipError_t launch_ln_quant(const void* x, int x_bf16, int64_t M, int64_t K, double ln_eps, float qb, float lim,
                           int layout, int8_t* q, int32_t* rowsum, float* stats, float* gamma_ws,
                           int8_t* xq_opt, float* gamma_opt, hipStream_t s) {
    if (x_bf16)
        launch_lnq_t(static_cast<const uint16_t*>(x), M, K, ln_eps, qb, lim, layout, q, rowsum, stats, gamma_ws,
                     xq_opt, gamma_opt, s);
    else
        launch_lnq_t(static_cast<const float*>(x), M, K, ln_eps, qb, lim, layout, q, rowsum, stats, gamma_ws,
                     xq_opt, gamma_opt, s);
    return hipGetLastError();
}

}  // namespace bgb
