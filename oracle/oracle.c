/*
 * CPU oracle for the binarized linear layers -- TEST INFRASTRUCTURE ONLY.
 * Only tests, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * Deliberately plain: one loop nest per definition, fp64 accumulation,
 * sums taken in ascending index order, no blocking and no threads.
 * See oracle.h for the sources; each function below names the passage it
 * follows. Build: gcc -O2 -std=c11 -ffp-contract=off (no fast-math).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- signs -- */

/* [BitNet] eq. (2): Sign(w) = +1 if w > 0, else -1 (zero and NaN go to -1).
 * [FBI-news]: FBI-linear binarizes the weights with the sign function; the
 * same tie rule is used. */
int oracle_sign_fbi(const float* W, int64_t K, int64_t N, int8_t* S) {
    if (!W || !S || K < 0 || N < 0) return -1;
    for (int64_t i = 0; i < K; ++i)
        for (int64_t j = 0; j < N; ++j)
            S[i * N + j] = (W[i * N + j] > 0.0f) ? 1 : -1;
    return 0;
}

/* [BitNet] eq. (1)-(2): W~ = Sign(W - c); the comparison W > c is the same
 * decision as W - c > 0 without the rounding of the subtraction. */
int oracle_sign_bitnet(const float* W, int64_t K, int64_t N, float c, int8_t* S) {
    if (!W || !S || K < 0 || N < 0) return -1;
    for (int64_t i = 0; i < K; ++i)
        for (int64_t j = 0; j < N; ++j)
            S[i * N + j] = (W[i * N + j] > c) ? 1 : -1;
    return 0;
}

/* ---------------------------------------------------------------- scales -- */

/* [FBI-news]: one full-precision scale per column, initialised from the
 * column average. Reading: alpha_j = (1/K) sum_i |W_ij| over the input index
 * i of output column j; fp64 sum, one fp64 division, rounded once to fp32. */
int oracle_fbi_alpha(const float* W, int64_t K, int64_t N, float* alpha) {
    if (!W || !alpha || K <= 0 || N < 0) return -1;
    for (int64_t j = 0; j < N; ++j) {
        double s = 0.0;
        for (int64_t i = 0; i < K; ++i) s += fabs((double)W[i * N + j]);
        alpha[j] = (float)(s / (double)K);
    }
    return 0;
}

/* [BitNet] eq. (3): c = (1/nm) sum_ij W_ij; eq. (8): beta = (1/nm) ||W||_1
 * (entrywise L1 norm of the uncentred W). fp64 sums, rounded once to fp32. */
int oracle_bitnet_scalars(const float* W, int64_t K, int64_t N, float* c, float* beta) {
    if (!W || !c || !beta || K <= 0 || N <= 0) return -1;
    double s = 0.0, a = 0.0;
    for (int64_t i = 0; i < K; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double w = (double)W[i * N + j];
            s += w;
            a += fabs(w);
        }
    double n = (double)K * (double)N;
    *c = (float)(s / n);
    *beta = (float)(a / n);
    return 0;
}

/* ---------------------------------------------------------------- packing -- */

/* The library's packed sign format (none is given on the pages, which only
 * say the weights take one bit each):
 *   K is a multiple of 32; T = K/32 words per column; TQ = ceil(T/4).
 *   The word for rows 32t..32t+31 of column j is at (t/4)*4N + 4j + (t%4).
 *   Bit b of that word is 1 iff sign(row 32t+b, column j) is +1.
 *   Words with t >= T are zero. */
int64_t oracle_packed_words(int64_t K, int64_t N) {
    if (K <= 0 || (K % 32) != 0 || N < 0) return -1;
    int64_t T = K / 32;
    int64_t TQ = (T + 3) / 4;
    return TQ * N * 4;
}

int oracle_pack(const int8_t* S, int64_t K, int64_t N, uint32_t* P) {
    int64_t words = oracle_packed_words(K, N);
    if (!S || !P || words < 0) return -1;
    memset(P, 0, (size_t)words * sizeof(uint32_t));
    for (int64_t i = 0; i < K; ++i) {
        int64_t t = i / 32;
        int b = (int)(i % 32);
        for (int64_t j = 0; j < N; ++j)
            if (S[i * N + j] > 0) P[(t / 4) * 4 * N + 4 * j + (t % 4)] |= (uint32_t)1u << b;
    }
    return 0;
}

/* ------------------------------------------------------- 16-bit formats -- */

/* IEEE binary16, round to nearest even, done in fp64 where every step is
 * exact except the single nearbyint (default rounding mode = to nearest even). */
uint16_t oracle_f32_to_f16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    double d = fabs((double)f);
    if (d != d) return (uint16_t)(sign | 0x7E00u);                 /* NaN */
    if (isinf(d)) return (uint16_t)(sign | 0x7C00u);               /* infinity */
    if (d < ldexp(1.0, -14)) {                                       /* subnormal range */
        double q = nearbyint(d * ldexp(1.0, 24));                    /* units of 2^-24 */
        return (uint16_t)(sign | (uint16_t)q);                       /* q == 1024 is the min normal */
    }
    int e2;
    frexp(d, &e2);                                                   /* d = m * 2^e2, m in [0.5,1) */
    int E = e2 - 1;                                                  /* d = 1.f * 2^E */
    double q = nearbyint(d * ldexp(1.0, 10 - E));                    /* 11-bit significand */
    if (q >= 2048.0) { q = 1024.0; E += 1; }
    if (E > 15) return (uint16_t)(sign | 0x7C00u);                   /* overflow -> inf */
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024.0));
}

float oracle_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int E = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    double v;
    if (E == 0) v = ldexp((double)frac, -24);
    else if (E == 31) v = frac ? NAN : INFINITY;
    else v = ldexp((double)(1024 + frac), E - 25);
    return (float)(sign ? -v : v);
}

float oracle_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ------------------------------------------------------------ FBI linear -- */

/* [FBI-news] W1A16: 1-bit weights (sign of W), 16-bit activations, output
 * column j scaled by alpha_j:  y[m][j] = alpha_j * sum_i s_ij * x[m][i].
 * fp64 throughout; each output is summed over i in ascending order. */
int oracle_fbi_linear(const uint16_t* x, int x_kind, int64_t M, int64_t K,
                      const float* W, int64_t N, const float* alpha, double* y) {
    if (!x || !W || !alpha || !y || M < 0 || K < 0 || N < 0) return -1;
    if (x_kind != 0 && x_kind != 1) return -1;
    for (int64_t m = 0; m < M; ++m) {
        double* row = y + m * N;
        for (int64_t j = 0; j < N; ++j) row[j] = 0.0;
        for (int64_t i = 0; i < K; ++i) {
            uint16_t xb = x[m * K + i];
            double xv = (double)(x_kind == 0 ? oracle_bf16_to_f32(xb) : oracle_f16_to_f32(xb));
            const float* wr = W + i * N;
            for (int64_t j = 0; j < N; ++j) row[j] += (wr[j] > 0.0f) ? xv : -xv;
        }
        for (int64_t j = 0; j < N; ++j) row[j] *= (double)alpha[j];
    }
    return 0;
}

/* [FBI-news], training paragraph: gradients pass the sign function through
 * the straight-through estimator, taken as the identity (no clipping is
 * stated). With y = alpha_j sum_i s_ij x_mi: dX = (dY * alpha) S^T,
 * dalpha_j = sum_m dY_mj z_mj with z = x S, and the gradient of W_b =
 * alpha * sign(W) passed to W, dW_ij = alpha_j sum_m x_mi dY_mj. One loop
 * nest per output, fp64, ascending index order. */
int oracle_fbi_backward(const uint16_t* x, const uint16_t* dy, int kind, int64_t M, int64_t K,
                        const float* W, int64_t N, const float* alpha, double* dx, double* dalpha,
                        double* dw) {
    if (M < 0 || K < 0 || N < 0 || !W || !alpha || !dy) return -1;
    if (kind != 0 && kind != 1) return -1;
    if ((dalpha || dw) && !x) return -1;
#define ORC_V16(b) ((double)(kind == 0 ? oracle_bf16_to_f32(b) : oracle_f16_to_f32(b)))
    if (dx) {
        for (int64_t m = 0; m < M; ++m)
            for (int64_t i = 0; i < K; ++i) {
                double acc = 0.0;
                for (int64_t j = 0; j < N; ++j) {
                    const double g = ORC_V16(dy[m * N + j]) * (double)alpha[j];
                    acc += (W[i * N + j] > 0.0f) ? g : -g;
                }
                dx[m * K + i] = acc;
            }
    }
    if (dalpha) {
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0;
            for (int64_t m = 0; m < M; ++m) {
                double z = 0.0;
                for (int64_t i = 0; i < K; ++i) {
                    const double xv = ORC_V16(x[m * K + i]);
                    z += (W[i * N + j] > 0.0f) ? xv : -xv;
                }
                acc += ORC_V16(dy[m * N + j]) * z;
            }
            dalpha[j] = acc;
        }
    }
    if (dw) {
        for (int64_t i = 0; i < K; ++i)
            for (int64_t j = 0; j < N; ++j) {
                double acc = 0.0;
                for (int64_t m = 0; m < M; ++m) acc += ORC_V16(x[m * K + i]) * ORC_V16(dy[m * N + j]);
                dw[i * N + j] = (double)alpha[j] * acc;
            }
    }
#undef ORC_V16
    return 0;
}

/* ------------------------------------------------------ BitLinear prologue -- */

/* [BitNet] eq. (8): LN(x) = (x - E(x)) / sqrt(Var(x) + eps), per token over K,
 * biased variance, no affine. eq. (4)-(5): Quant(x) = Clip(x * Q_b / gamma,
 * -Q_b + eps, Q_b - eps) with gamma = ||x||_inf over the input matrix and
 * Q_b = 2^(b-1).
 *
 * Readings (the pages leave these open):
 *  - E(x) and Var(x) are computed in fp64 (two passes), then mu32 = fl32(E(x))
 *    and rstd32 = fl32(1/sqrt(Var(x) + eps)).
 *  - The quantized code is an integer decided by floating point, so it is
 *    decided in fp32, the device's precision:
 *        h = fl32(fl32(x - mu32) * rstd32)
 *        gamma = max |h| over all M*K entries (exact)
 *        v = fl32((h * Q_b) / gamma)     (h * Q_b is exact: Q_b is a power of 2)
 *        lim = fl32(Q_b - q_eps);  v_c = min(lim, max(-lim, v))
 *        q = trunc(v_c)  (toward zero: the only rounding under which eps keeps
 *                         q inside [-(Q_b-1), Q_b-1], its stated purpose)
 *  - gamma == 0 (every h is zero) gives q == 0. */
int oracle_ln_absmax_quant(const float* x, int64_t M, int64_t K, double ln_eps, int bits,
                           float q_eps, int round_mode, int gamma_scope, int8_t* q, float* gamma,
                           float* mu32, float* rstd32) {
    if (!x || !q || !gamma || M < 0 || K <= 0 || bits < 2 || bits > 8) return -1;
    if (round_mode < 0 || round_mode > 1 || gamma_scope < 0 || gamma_scope > 1) return -1;
    const float Qb = (float)(1 << (bits - 1));
    const int qmax = (1 << (bits - 1)) - 1;
    const size_t nm = (size_t)(M > 0 ? M : 1);
    float* mu_f = (float*)malloc(sizeof(float) * nm);
    float* rs_f = (float*)malloc(sizeof(float) * nm);
    float* gm = (float*)malloc(sizeof(float) * nm);
    if (!mu_f || !rs_f || !gm) { free(mu_f); free(rs_f); free(gm); return -2; }
    /* statistics per token; each token's max |h|, then gamma over the tensor */
    float g = 0.0f;
    for (int64_t m = 0; m < M; ++m) {
        const float* xr = x + m * K;
        double s = 0.0;
        for (int64_t i = 0; i < K; ++i) s += (double)xr[i];
        double mu = s / (double)K;
        double v2 = 0.0;
        for (int64_t i = 0; i < K; ++i) {
            double d = (double)xr[i] - mu;
            v2 += d * d;
        }
        double var = v2 / (double)K;
        mu_f[m] = (float)mu;
        rs_f[m] = (float)(1.0 / sqrt(var + ln_eps));
        float rowmax = 0.0f;
        for (int64_t i = 0; i < K; ++i) {
            float d = xr[i] - mu_f[m];
            float h = d * rs_f[m];
            float a = fabsf(h);
            if (a > rowmax) rowmax = a;
        }
        gm[m] = rowmax;
        if (rowmax > g) g = rowmax;
    }
    if (gamma_scope == 0) gamma[0] = g;
    /* quantize with the token's gamma (scope 1) or the tensor's (scope 0) */
    const float lim = Qb - q_eps;
    for (int64_t m = 0; m < M; ++m) {
        const float* xr = x + m * K;
        const float gr = gamma_scope == 1 ? gm[m] : g;
        if (gamma_scope == 1) gamma[m] = gr;
        for (int64_t i = 0; i < K; ++i) {
            if (gr == 0.0f) { q[m * K + i] = 0; continue; }
            float d = xr[i] - mu_f[m];
            float h = d * rs_f[m];
            float v = (h * Qb) / gr;
            float vc = v > lim ? lim : (v < -lim ? -lim : v);
            int c;
            if (round_mode == 0) {
                c = (int)vc;                       /* toward zero */
            } else {
                c = (int)nearbyintf(vc);           /* nearest, ties to even (default FP environment) */
                if (c > qmax) c = qmax;
                if (c < -qmax) c = -qmax;
            }
            q[m * K + i] = (int8_t)c;
        }
        if (mu32) mu32[m] = mu_f[m];
        if (rstd32) rstd32[m] = rs_f[m];
    }
    free(mu_f);
    free(rs_f);
    free(gm);
    return 0;
}

/* [BitNet] eq. (6): for activations ahead of a non-linear function the codes
 * are shifted to be non-negative: Quant(x) = Clip((x - eta) Q_b / gamma,
 * eps, Q_b - eps) with eta = min x. Readings: x is the LayerNorm output h
 * (eq. (7) quantizes LN(x)); gamma keeps its one definition, eq. (5),
 * ||h||_inf; eta and gamma are taken over the tensor (scope 0) or the token
 * (scope 1). Decided in fp32 like eq. (4): d = fl32(h - eta),
 * v = fl32((d * Q_b) / gamma), v_c = min(fl32(Q_b - eps), max(fl32(eps), v)),
 * then truncation (or round to nearest even, clamped to Q_b - 1); gamma == 0
 * (every h zero) gives q == 0. eta: [1] or [M]. */
int oracle_ln_nonneg_quant(const float* x, int64_t M, int64_t K, double ln_eps, int bits, float q_eps,
                           int round_mode, int gamma_scope, int8_t* q, float* gamma, float* eta) {
    if (!x || !q || !gamma || !eta || M < 0 || K <= 0 || bits < 2 || bits > 8) return -1;
    if (round_mode < 0 || round_mode > 1 || gamma_scope < 0 || gamma_scope > 1) return -1;
    const float Qb = (float)(1 << (bits - 1));
    const int qmax = (1 << (bits - 1)) - 1;
    const size_t n = (size_t)(M > 0 ? M : 1) * (size_t)K;
    float* h = (float*)malloc(sizeof(float) * n);
    if (!h) return -2;
    /* LayerNorm per token (fp64 statistics, fp32 application), as for eq. (4) */
    for (int64_t m = 0; m < M; ++m) {
        const float* xr = x + m * K;
        double s = 0.0;
        for (int64_t i = 0; i < K; ++i) s += (double)xr[i];
        const double mu = s / (double)K;
        double v2 = 0.0;
        for (int64_t i = 0; i < K; ++i) {
            const double d = (double)xr[i] - mu;
            v2 += d * d;
        }
        const float mu32 = (float)mu;
        const float rs32 = (float)(1.0 / sqrt(v2 / (double)K + ln_eps));
        for (int64_t i = 0; i < K; ++i) {
            const float d = xr[i] - mu32;
            h[m * K + i] = d * rs32;
        }
    }
    const float lo = q_eps, hi = Qb - q_eps;
    for (int64_t m = 0; m < M; ++m) {
        /* the scope's gamma = max |h| and eta = min h */
        const int64_t b = gamma_scope == 1 ? m * K : 0, e = gamma_scope == 1 ? (m + 1) * K : M * K;
        float g = 0.0f, mn = h[b];
        for (int64_t i = b; i < e; ++i) {
            const float a = fabsf(h[i]);
            if (a > g) g = a;
            if (h[i] < mn) mn = h[i];
        }
        if (gamma_scope == 1) {
            gamma[m] = g;
            eta[m] = mn;
        } else if (m == 0) {
            gamma[0] = g;
            eta[0] = mn;
        }
        for (int64_t i = 0; i < K; ++i) {
            if (g == 0.0f) { q[m * K + i] = 0; continue; }
            const float d = h[m * K + i] - mn;
            const float v = (d * Qb) / g;
            const float vc = v > hi ? hi : (v < lo ? lo : v);
            int c = round_mode == 0 ? (int)vc : (int)nearbyintf(vc);
            if (c > qmax) c = qmax;
            q[m * K + i] = (int8_t)c;
        }
    }
    free(h);
    return 0;
}

/* ------------------------------------------------------- BitLinear product -- */

/* [BitNet] eq. (7): the integer part W~ . Quant(LN(x)), with W~ = Sign(W - c).
 * Exact in int64, summed over i in ascending order. */
int oracle_bitlinear_acc(const int8_t* q, int64_t M, int64_t K, const float* W, int64_t N,
                         float c, int64_t* acc) {
    if (!q || !W || !acc || M < 0 || K < 0 || N < 0) return -1;
    for (int64_t m = 0; m < M; ++m) {
        int64_t* row = acc + m * N;
        for (int64_t j = 0; j < N; ++j) row[j] = 0;
        for (int64_t i = 0; i < K; ++i) {
            int64_t qv = q[m * K + i];
            const float* wr = W + i * N;
            for (int64_t j = 0; j < N; ++j) row[j] += (wr[j] > c) ? qv : -qv;
        }
    }
    return 0;
}

/* [BitNet] eq. (7): y = W~ Quant(LN(x)) * beta * gamma / Q_b, in fp64. */
int oracle_bitlinear_out(const int64_t* acc, int64_t M, int64_t N, float beta, float gamma,
                         int bits, double* y) {
    if (!acc || !y || M < 0 || N < 0 || bits < 2 || bits > 8) return -1;
    double Qb = (double)(1 << (bits - 1));
    for (int64_t i = 0; i < M * N; ++i)
        y[i] = (double)acc[i] * (double)beta * (double)gamma / Qb;
    return 0;
}

/* ------------------------------------------------- BitNet b1.58 (ternary) -- */

/* [BitNet] section 二, eq. (9)-(11). The page leaves the rounding of round()
 * and the value of eps open; round to nearest even is taken, eps is an input. */
int oracle_ternary(const float* W, int64_t K, int64_t N, float eps_w, int8_t* T, float* gamma_w) {
    if (!W || !T || !gamma_w || K <= 0 || N <= 0 || !(eps_w >= 0.0f)) return -1;
    double a = 0.0;
    for (int64_t i = 0; i < K; ++i)
        for (int64_t j = 0; j < N; ++j) a += fabs((double)W[i * N + j]);
    const float g = (float)(a / ((double)K * (double)N));   /* eq. (11) */
    const float den = g + eps_w;                              /* gamma + eps in fp32 */
    for (int64_t i = 0; i < K; ++i)
        for (int64_t j = 0; j < N; ++j) {
            float t = W[i * N + j] / den;                     /* eq. (9), fp32 quotient */
            float r = nearbyintf(t);                          /* round, ties to even */
            T[i * N + j] = (int8_t)(r > 1.0f ? 1 : (r < -1.0f ? -1 : (int)r));   /* eq. (10) clip */
        }
    *gamma_w = g;
    return 0;
}

int oracle_int8_acc(const int8_t* q, int64_t M, int64_t K, const int8_t* T, int64_t N, int64_t* acc) {
    if (!q || !T || !acc || M < 0 || K < 0 || N < 0) return -1;
    for (int64_t m = 0; m < M; ++m) {
        int64_t* row = acc + m * N;
        for (int64_t j = 0; j < N; ++j) row[j] = 0;
        for (int64_t i = 0; i < K; ++i) {
            const int64_t qi = q[m * K + i];
            const int8_t* trow = T + i * N;
            for (int64_t j = 0; j < N; ++j) row[j] += (int64_t)trow[j] * qi;
        }
    }
    return 0;
}
