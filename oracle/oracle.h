/*
 * CPU oracle for the binarized linear layers -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded reference written from the pages'
 * definitions. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the library's compute path never does.
 * It shares no code, header or table with the device library.
 *
 * Sources (by page title and passage):
 *   [FBI-news]  "FBI-LLM ... An AI Framework Utilizing Autoregressive Distillation
 *               for 1-bit Weight Binarization of LLMs from Scratch", the paragraph
 *               introducing FBI-linear (sign binarization, full-precision
 *               per-column scale initialised from column averages) and the
 *               experiments paragraph (W1A16).
 *   [BitNet]    "BitNet b1.58: 1bit LLM时代" blog, section 一 (BitNet):
 *               eq. (1)-(3) weight binarization, eq. (4)-(5) absmax quant,
 *               eq. (7)-(8) BitLinear output, LayerNorm and beta.
 *
 * Layout conventions: W is float32 [K][N] row-major (row i = input feature,
 * column j = output feature); activations are [M][K]; outputs [M][N].
 * All functions return 0 on success and a negative value on bad arguments.
 */
#ifndef BGB_ORACLE_H
#define BGB_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Sign with ties to -1 ([BitNet] eq. (2)); FBI-linear takes the sign of W itself. */
int oracle_sign_fbi(const float* W, int64_t K, int64_t N, int8_t* S);
/* BitNet: sign of (W - c), again with ties to -1 ([BitNet] eq. (1)-(2)). */
int oracle_sign_bitnet(const float* W, int64_t K, int64_t N, float c, int8_t* S);

/* FBI per-output-column scale: alpha_j = mean_i |W_ij|, fp64 sum rounded once to fp32. */
int oracle_fbi_alpha(const float* W, int64_t K, int64_t N, float* alpha);
/* BitNet centre c = mean(W) ([BitNet] eq. (3)) and beta = ||W||_1/(KN) ([BitNet] eq. (8)). */
int oracle_bitnet_scalars(const float* W, int64_t K, int64_t N, float* c, float* beta);

/* Packed sign format: number of uint32 words, and the packing itself. */
int64_t oracle_packed_words(int64_t K, int64_t N);
int oracle_pack(const int8_t* S, int64_t K, int64_t N, uint32_t* P);

/* IEEE binary16 conversions (round to nearest even) used for stored scales. */
uint16_t oracle_f32_to_f16(float f);
float oracle_f16_to_f32(uint16_t h);
float oracle_bf16_to_f32(uint16_t b);

/* FBI-linear W1A16: y[m][j] = alpha_j * sum_i sign(W_ij) * x[m][i], in fp64.
 * x_kind: 0 = bf16 bits, 1 = f16 bits. alpha is the stored scale widened to float. */
int oracle_fbi_linear(const uint16_t* x, int x_kind, int64_t M, int64_t K,
                      const float* W, int64_t N, const float* alpha, double* y);

/* FBI-linear backward through the straight-through estimator ([FBI-news],
 * training paragraph: the STE carries gradients through the sign function).
 * Given dY [M][N] (16-bit, bit patterns of the same kind as x):
 *   dX[m][i]  = sum_j dY[m][j] alpha_j s_ij                       [M][K]
 *   dalpha_j  = sum_m dY[m][j] z[m][j],  z = x S (unscaled forward) [N]
 *   dW[i][j]  = alpha_j sum_m x[m][i] dY[m][j]                    [K][N]
 * (dW: the gradient reaching W_b = alpha * sign(W), passed through sign as
 * the identity, since the pages state no clipping). fp64; any output may be
 * NULL. */
int oracle_fbi_backward(const uint16_t* x, const uint16_t* dy, int kind, int64_t M, int64_t K,
                        const float* W, int64_t N, const float* alpha, double* dx, double* dalpha,
                        double* dw);

/* BitLinear prologue: per-token LayerNorm (no affine), then absmax quantization to
 * [-Q_b+eps, Q_b-eps] with Q_b = 2^(bits-1), gamma = max |LN(x)| over the tensor.
 * Statistics in fp64; the quantization decision in fp32 (see oracle.c).
 * round_mode: 0 = truncate toward zero (the reading of eq. (4)), 1 = round to
 * nearest even, then clamp to +-(Q_b - 1). gamma_scope: 0 = one gamma over the
 * whole tensor (the reading of section 一), 1 = one gamma per token.
 * Outputs: q [M][K], gamma ([1] for scope 0, [M] for scope 1), and per-row
 * mu32/rstd32 (optional, may be NULL). */
int oracle_ln_absmax_quant(const float* x, int64_t M, int64_t K, double ln_eps, int bits,
                           float q_eps, int round_mode, int gamma_scope, int8_t* q, float* gamma,
                           float* mu32, float* rstd32);

/* [BitNet] eq. (6): the non-negative quantizer, codes in [0, Q_b - 1]:
 * q = Clip((h - eta) Q_b / gamma, eps, Q_b - eps) with h = LN(x) as above,
 * gamma = max |h| (eq. (5)) and eta = min h over the tensor (scope 0) or the
 * token (scope 1); fp32 decisions, truncation or round to nearest even.
 * gamma, eta: [1] or [M]. */
int oracle_ln_nonneg_quant(const float* x, int64_t M, int64_t K, double ln_eps, int bits, float q_eps,
                           int round_mode, int gamma_scope, int8_t* q, float* gamma, float* eta);

/* BitLinear integer product acc[m][j] = sum_i sign(W_ij - c) * q[m][i] (exact). */
int oracle_bitlinear_acc(const int8_t* q, int64_t M, int64_t K, const float* W, int64_t N,
                         float c, int64_t* acc);
/* BitNet b1.58 ternary weights ([BitNet] section 二, eq. (9)-(11)):
 * gamma_w = mean |W| (fp64 sum rounded once to fp32), then
 * T_ij = RoundClip(W_ij / (gamma_w + eps_w), -1, 1): the divisor and the
 * quotient in fp32, round to nearest even, clip to [-1, 1]. */
int oracle_ternary(const float* W, int64_t K, int64_t N, float eps_w, int8_t* T, float* gamma_w);

/* Integer product acc[m][j] = sum_i T_ij * q[m][i] for int8 weights T [K][N]
 * (the ternary BitLinear product), exact in int64, i ascending. */
int oracle_int8_acc(const int8_t* q, int64_t M, int64_t K, const int8_t* T, int64_t N, int64_t* acc);

/* BitLinear output y = acc * beta * gamma / Q_b in fp64 ([BitNet] eq. (7)). */
int oracle_bitlinear_out(const int64_t* acc, int64_t M, int64_t N, float beta, float gamma,
                         int bits, double* y);

#ifdef __cplusplus
}
#endif
#endif
