// BitLinear prologue: per-token LayerNorm, tensor-wide absmax, b-bit codes.
//
// "BitNet b1.58: 1bit LLM时代" blog, section 一 (BitNet): eq. (8) LayerNorm
// (x - E x) / sqrt(Var x + eps); eq. (4)-(5) Quant(x) = Clip(x Q_b / gamma,
// -Q_b + eps, Q_b - eps) with gamma = ||x||_inf over the input matrix.
//
// Numerics (fixed so that codes are reproducible and identical to the
// reference): E x and Var x (biased, two passes) in fp64; mu32 = fl32(E x),
// rstd32 = fl32(1 / sqrt(Var x + eps)); h = fl32(fl32(x - mu32) * rstd32);
// gamma = max |h| (over the tensor, or per token as an option);
// v = fl32(h Q_b / gamma) (h Q_b exact, one rounding); clip to +-lim with
// lim = fl32(Q_b - q_eps); truncate toward zero (or, as an option, round to
// nearest even and clamp to +-(Q_b - 1)).
//
// The non-negative range (eq. (6), for activations ahead of a non-linear
// function): the codes are Clip((h - eta) Q_b / gamma, eps, Q_b - eps) with
// eta = min h over the same scope as gamma (which keeps eq. (5)'s
// definition), decided in fp32 as d = fl32(h - eta), v = fl32(d Q_b / gamma);
// codes lie in [0, Q_b - 1]. The product and eq. (7)'s output are unchanged.
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

BGB_DEV int quant_code(float h, float qb, float gamma, float lim, bool rne, int qmax) {
    if (gamma == 0.0f) return 0;
    float v = (h * qb) / gamma;
    v = fminf(fmaxf(v, -lim), lim);
    return round_code(v, rne, qmax);
}

// eq. (6): d = fl32(h - eta) >= 0; the lower clip at eps never changes a code.
BGB_DEV int quant_code_nn(float d, float qb, float gamma, float lo, float lim, bool rne, int qmax) {
    if (gamma == 0.0f) return 0;
    float v = (d * qb) / gamma;
    v = fminf(fmaxf(v, lo), lim);
    return round_code(v, rne, qmax);
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
                      float lim, bool rne, bool nonneg, float eta, float lo, int layout, uint32_t* qrow,
                      int8_t* natrow, int* iscr) {
    const int qmax = int(qb) - 1;
    int sum = 0;
    for (int64_t dwi = threadIdx.x; dwi < Kp / 4; dwi += NT) {
        const int64_t k0 = (dwi / 32) * 128 + code_base(layout, int(dwi % 32));
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t k = k0 + 8 * e;
            int c = 0;
            if (k < K) {
                const float h = ln_apply(load_x(xr, k), mu32, rs32);
                c = nonneg ? quant_code_nn(h - eta, qb, gamma, lo, lim, rne, qmax)
                           : quant_code(h, qb, gamma, lim, rne, qmax);
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
                 int rne, int token, int nonneg, float lo, int layout, int8_t* __restrict__ q,
                 int32_t* __restrict__ rowsum,
                 float* __restrict__ stats, float* __restrict__ gamma_ws, int8_t* __restrict__ xq_opt,
                 float* __restrict__ gamma_opt) {
    __shared__ double dscr[16];
    __shared__ float fscr[16];
    __shared__ int iscr[16];
    __shared__ float s_mu[kSmallPrologueM], s_rs[kSmallPrologueM], s_lm[kSmallPrologueM], s_mn[kSmallPrologueM];
    float gmax = 0.0f, gmin = __builtin_inff();
    for (int m = 0; m < M; ++m) {
        const XT* xr = x + int64_t(m) * K;
        float mu32, rs32;
        row_stats<1024>(xr, K, eps, dscr, mu32, rs32);
        float lm = 0.0f;
        for (int64_t i = threadIdx.x; i < K; i += 1024) lm = fmaxf(lm, fabsf(ln_apply(load_x(xr, i), mu32, rs32)));
        lm = block_max<1024>(lm, fscr);
        float mn = __builtin_inff();                 // eq. (6): the row's min h (min x, h monotone in x)
        if (nonneg) {
            for (int64_t i = threadIdx.x; i < K; i += 1024) mn = fminf(mn, ln_apply(load_x(xr, i), mu32, rs32));
            mn = -block_max<1024>(-mn, fscr);
        }
        if (threadIdx.x == 0) {
            s_mu[m] = mu32;
            s_rs[m] = rs32;
            s_lm[m] = lm;
            s_mn[m] = mn;
            stats[3 * m] = mu32;
            stats[3 * m + 1] = rs32;
            stats[3 * m + 2] = lm;
        }
        gmax = fmaxf(gmax, lm);
        gmin = fminf(gmin, mn);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        gamma_ws[0] = gmax;
        if (gamma_opt && !token) gamma_opt[0] = gmax;
    }
    if (gamma_opt && token && threadIdx.x < M) gamma_opt[threadIdx.x] = s_lm[threadIdx.x];
    for (int m = 0; m < M; ++m) {
        const float gamma = token ? s_lm[m] : gmax;     // the token's own, or the tensor's
        const float eta = token ? s_mn[m] : gmin;
        const int s = quant_row<1024>(x + int64_t(m) * K, K, Kp, s_mu[m], s_rs[m], qb, gamma, lim, rne != 0,
                                      nonneg != 0, eta, lo, layout,
                                      reinterpret_cast<uint32_t*>(q + int64_t(m) * Kp),
                                      xq_opt ? xq_opt + int64_t(m) * K : nullptr, iscr);
        if (threadIdx.x == 0) rowsum[m] = s;
    }
}

// Large M: one wave per row, four rows per block, rows read in 16-byte
// vectors (K % 32 == 0 keeps every row 16-byte aligned).
template <typename XT> struct Vec16;
template <> struct Vec16<float> {            // 4 elements per 16 bytes
    static constexpr int E = 4;
    static BGB_DEV void load(const float* p, float* v) {
        const f32x4_t t = *reinterpret_cast<const f32x4_t*>(p);
        v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
    }
};
template <> struct Vec16<uint16_t> {         // 8 bf16 elements per 16 bytes
    static constexpr int E = 8;
    static BGB_DEV void load(const uint16_t* p, float* v) {
        const u32x4_t t = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(t[i] << 16);
            v[2 * i + 1] = __uint_as_float(t[i] & 0xffff0000u);
        }
    }
};

// Pass 1: mu32, rstd32 and max |h| of each row (|h| is largest at the row's
// largest or smallest x, h being monotone in x), and the max over the
// block's rows for pass 2.
template <typename XT>
__global__ void __launch_bounds__(256)
lnq_stats_kernel(const XT* __restrict__ x, int64_t M, int64_t K, double eps, float* __restrict__ stats,
                 float* __restrict__ blockmax, float* __restrict__ mins) {
    using V = Vec16<XT>;
    constexpr int E = V::E;
    __shared__ float bm[4], bn[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m = int64_t(blockIdx.x) * 4 + wave;
    float rowmax = 0.0f, rowmin = __builtin_inff();
    if (m < M) {
        const XT* xr = x + m * K;
        const int64_t nvec = K / E;
        double s = 0.0;
        float mx = -__builtin_inff(), mn = __builtin_inff();
        for (int64_t c = lane; c < nvec; c += 64) {
            float v[E];
            V::load(xr + c * E, v);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                s += double(v[e]);
                mx = fmaxf(mx, v[e]);
                mn = fminf(mn, v[e]);
            }
        }
        s = wave_sum63(s);
        mx = wave_max63(mx);
        mn = wave_min63(mn);
        const double mu = __shfl(s, 63) / double(K);
        double s2 = 0.0;
        for (int64_t c = lane; c < nvec; c += 64) {
            float v[E];
            V::load(xr + c * E, v);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const double d = double(v[e]) - mu;
                s2 += d * d;
            }
        }
        s2 = wave_sum63(s2);
        const float mu32 = float(mu);
        const float rs32 = float(1.0 / sqrt(__shfl(s2, 63) / double(K) + eps));
        const float hx = __shfl(mx, 63), hn = __shfl(mn, 63);
        rowmax = fmaxf(fabsf(ln_apply(hx, mu32, rs32)), fabsf(ln_apply(hn, mu32, rs32)));
        rowmin = ln_apply(hn, mu32, rs32);                  // h is monotone in x
        if (mins && lane == 0) mins[m] = rowmin;
        if (lane == 0) {
            stats[3 * m] = mu32;
            stats[3 * m + 1] = rs32;
            stats[3 * m + 2] = rowmax;
        }
    }
    if (lane == 0) {
        bm[wave] = rowmax;
        bn[wave] = rowmin;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        blockmax[blockIdx.x] = fmaxf(fmaxf(bm[0], bm[1]), fmaxf(bm[2], bm[3]));
        if (mins) mins[M + blockIdx.x] = fminf(fminf(bn[0], bn[1]), fminf(bn[2], bn[3]));
    }
}

// Pass 2: gamma = max over the block maxima (every block computes the same
// exact value), then one wave per row: lane t takes 32-row words t, t + 64,
// ..., computes their 32 codes and stores the 8 code dwords of the word in
// the requested layout (zeros for the padding words past K).
template <typename XT>
__global__ void __launch_bounds__(256)
lnq_quant_kernel(const XT* __restrict__ x, int64_t M, int64_t K, int64_t Kp, float qb, float lim, int rne,
                 int token, float lo, int layout, const float* __restrict__ stats, const float* __restrict__ blockmax,
                 const float* __restrict__ mins, int nblocks,
                 int8_t* __restrict__ q, int32_t* __restrict__ rowsum, float* __restrict__ gamma_ws,
                 int8_t* __restrict__ xq_opt, float* __restrict__ gamma_opt) {
    using V = Vec16<XT>;
    constexpr int E = V::E;
    __shared__ float gscr[4], nscr[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float gm = 0.0f, gn = __builtin_inff();
    for (int i = threadIdx.x; i < nblocks; i += 256) {
        gm = fmaxf(gm, blockmax[i]);
        if (mins) gn = fminf(gn, mins[M + i]);
    }
    gm = wave_max63_nonneg(gm);
    gn = wave_min63(gn);
    if (lane == 63) {
        gscr[wave] = gm;
        nscr[wave] = gn;
    }
    __syncthreads();
    const float gt = fmaxf(fmaxf(gscr[0], gscr[1]), fmaxf(gscr[2], gscr[3]));
    const float nt = fminf(fminf(nscr[0], nscr[1]), fminf(nscr[2], nscr[3]));
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        gamma_ws[0] = gt;
        if (gamma_opt && !token) gamma_opt[0] = gt;
    }
    const int64_t m = int64_t(blockIdx.x) * 4 + wave;
    if (m >= M) return;
    const XT* xr = x + m * K;
    const float mu32 = stats[3 * m], rs32 = stats[3 * m + 1];
    const float gamma = token ? stats[3 * m + 2] : gt;      // the token's own, or the tensor's
    const bool nonneg = mins != nullptr;
    const float eta = nonneg ? (token ? mins[m] : nt) : 0.0f;
    if (gamma_opt && token && lane == 0) gamma_opt[m] = gamma;
    const bool rn = rne != 0;
    const float cq = gamma != 0.0f ? qb * __builtin_amdgcn_rcpf(gamma) : 0.0f;
    // gamma below about Q_b / FLT_MAX overflows Q_b rcp(gamma): no fast quotient
    // is meaningful then, and every code comes from the exact division
    const uint32_t all_slow = cq <= 0x1.fffffep127f ? 0u : 0xffffffffu;
    const int qmax = int(qb) - 1;
    const int64_t words = K / 32, pwords = Kp / 32;
    int sum = 0;
    for (int64_t t = lane; t < pwords; t += 64) {
        uint32_t dw[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        if (t < words) {
            float h[32];
#pragma unroll
            for (int c = 0; c < 32 / E; ++c) V::load(xr + 32 * t + c * E, h + c * E);
            int code[32];
            uint32_t slow = all_slow;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                h[j] = ln_apply(h[j], mu32, rs32);
                if (nonneg) h[j] = h[j] - eta;               // eq. (6): d = fl32(h - eta)
                // fast path: u = h (Q_b rcp(gamma)) is within 1.5 ulp of the exact
                // quotient; only u near a code boundary (rare) can round differently
                const float u = h[j] * cq;
                slow |= uint32_t(code_near_boundary(u, rn)) << j;
                code[j] = round_code(u, rn, qmax);
            }
            if (slow && gamma != 0.0f) {
#pragma unroll
                for (int j = 0; j < 32; ++j)
                    if (slow & (1u << j))
                        code[j] = nonneg ? quant_code_nn(h[j], qb, gamma, lo, lim, rn, qmax)
                                         : quant_code(h[j], qb, gamma, lim, rn, qmax);
            }
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                sum += code[j];
                dw[j & 7] |= uint32_t(uint8_t(int8_t(code[j]))) << (8 * (j >> 3));   // rows w + 8e of dword w
            }
            if (xq_opt) {
                u32x4_t nat[2];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    nat[i >> 2][i & 3] = uint32_t(uint8_t(int8_t(code[4 * i]))) | uint32_t(uint8_t(int8_t(code[4 * i + 1]))) << 8 |
                                         uint32_t(uint8_t(int8_t(code[4 * i + 2]))) << 16 |
                                         uint32_t(uint8_t(int8_t(code[4 * i + 3]))) << 24;
                u32x4_t* dst = reinterpret_cast<u32x4_t*>(xq_opt + m * K + 32 * t);
                dst[0] = nat[0];
                dst[1] = nat[1];
            }
        }
        int8_t* tile = q + m * Kp + (t >> 2) * 128;
        const int d = int(t & 3);
        if (layout == 1) {           // GEMM: dword 8d + w
            u32x4_t* dst = reinterpret_cast<u32x4_t*>(tile + 32 * d);
            dst[0] = u32x4_t{dw[0], dw[1], dw[2], dw[3]};
            dst[1] = u32x4_t{dw[4], dw[5], dw[6], dw[7]};
        } else {                     // decode: dword 4w + d
            uint32_t* dst = reinterpret_cast<uint32_t*>(tile);
#pragma unroll
            for (int w = 0; w < 8; ++w) dst[4 * w + d] = dw[w];
        }
    }
    sum = wave_sum63_i(sum);
    if (lane == 63) rowsum[m] = sum;
}

template <typename XT>
static void launch_lnq_t(const XT* x, int64_t M, int64_t K, double eps, float qb, float lim, int rne, int token,
                         float* mins, float lo, int layout, int8_t* q, int32_t* rowsum, float* stats,
                         float* gamma_ws, int8_t* xq_opt, float* gamma_opt, hipStream_t s) {
    const int64_t Kp = padded_k(K);
    if (M <= kSmallPrologueM) {
        lnq_small_kernel<XT><<<1, 1024, 0, s>>>(x, int(M), K, Kp, eps, qb, lim, rne, token, mins != nullptr, lo,
                                                 layout, q, rowsum, stats, gamma_ws, xq_opt, gamma_opt);
    } else {
        const unsigned blocks = unsigned((M + 3) / 4);
        float* blockmax = stats + 3 * M;       // the workspace's stats region holds [M][3] + ceil(M/4)
        lnq_stats_kernel<XT><<<blocks, 256, 0, s>>>(x, M, K, eps, stats, blockmax, mins);
        lnq_quant_kernel<XT><<<blocks, 256, 0, s>>>(x, M, K, Kp, qb, lim, rne, token, lo, layout, stats, blockmax,
                                                     mins, int(blocks), q, rowsum, gamma_ws, xq_opt, gamma_opt);
    }
}

hipError_t launch_ln_quant(const void* x, int x_bf16, int64_t M, int64_t K, double ln_eps, float qb, float lim,
                           int rne, int token, float* mins, float lo, int layout, int8_t* q, int32_t* rowsum,
                           float* stats, float* gamma_ws, int8_t* xq_opt, float* gamma_opt, hipStream_t s) {
    if (x_bf16)
        launch_lnq_t(static_cast<const uint16_t*>(x), M, K, ln_eps, qb, lim, rne, token, mins, lo, layout, q, rowsum,
                     stats, gamma_ws, xq_opt, gamma_opt, s);
    else
        launch_lnq_t(static_cast<const float*>(x), M, K, ln_eps, qb, lim, rne, token, mins, lo, layout, q, rowsum,
                     stats, gamma_ws, xq_opt, gamma_opt, s);
    return hipGetLastError();
}

}  // namespace bgb
