/*
 * bgb.h -- C ABI of the binarized linear layer library (libbgb.so, gfx950).
 *
 * Two layers are provided, each as a one-time weight conversion plus a
 * forward pass:
 *
 *   FBI-linear (W1A16), from "FBI-LLM ... An AI Framework Utilizing
 *   Autoregressive Distillation for 1-bit Weight Binarization of LLMs from
 *   Scratch" (news rewrite of the FBI-LLM paper), paragraph introducing
 *   FBI-linear: weights binarized with the sign function, one full-precision
 *   scale per column initialised from the column average, 16-bit activations
 *   (the W1A16 setting of its experiments paragraph).
 *
 *   BitLinear (W1A8), from the "BitNet b1.58: 1bit LLM时代" blog, section 一
 *   (BitNet): eq. (1)-(3) zero-centred sign binarization, eq. (4)-(5) absmax
 *   activation quantization, eq. (7)-(8) output rescale, LayerNorm and beta.
 *   "BitNet-Transformers: 1比特量化技术在大型语言模型中的应用与实现" presents
 *   BitLinear as a drop-in replacement for a linear layer, which fixes the
 *   shape of this interface: a conversion step plus a forward call.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Shapes: W is float32 [K][N] row-major (row i = input feature, column j =
 *   output feature); activations x are [M][K]; outputs y are [M][N]; all
 *   row-major and contiguous. y = x . W_b (scaled), i.e. the same product as
 *   a linear layer with in_features = K and out_features = N.
 * - K must be a positive multiple of 32. M == 0 or N == 0 is a valid empty
 *   call that launches nothing (its array pointers may then be NULL; shapes,
 *   dtypes and parameters are still checked). Limits: K <= 524288, M <= 2^24, N <= 2^24,
 *   and M*K, K*N, M*N each < 2^31 elements.
 * - Every pointer argument is a DEVICE pointer on the current HIP device,
 *   16-byte aligned, owned by the caller. The library allocates nothing and
 *   keeps no state between calls except the last HIP error code.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream). Nothing is copied back to the host. Results are bit-identical
 *   from run to run (fixed reduction orders, no floating-point atomics).
 * - Scratch memory comes from the caller's workspace `ws` of `ws_bytes`
 *   bytes (256-byte aligned); bgb_workspace_bytes() gives the size needed.
 *   Calls that share a workspace must be ordered (same stream).
 * - Errors: 0 on success, else a negative bgb_status. Arguments are
 *   validated before any launch; a rejected call writes no output.
 *
 * Packed sign format P (the pages only say each weight takes one bit):
 *   T = K/32 words per column, TQ = ceil(T/4); P holds TQ*N*4 uint32 words
 *   (bgb_packed_bytes). The word covering rows 32t..32t+31 of column j sits
 *   at index (t/4)*4N + 4j + (t%4), so each column's 128 consecutive rows
 *   form one 16-byte tile and the tiles of one 128-row band are stored column
 *   after column. Bit b (LSB = 0) of that word is 1 iff the sign of weight
 *   (row 32t+b, column j) is +1, 0 iff it is -1. Words with t >= T are 0.
 */
#ifndef BGB_H
#define BGB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BGB_OK = 0,
    BGB_EINVAL = -1,        /* null pointer, bad shape, misalignment, small workspace */
    BGB_EUNSUPPORTED = -2,  /* dtype or mode combination not implemented */
    BGB_EHIP = -3,          /* a HIP launch failed; see bgb_last_hip_error() */
    BGB_ESCRATCH = -4       /* bitlinear_w1a8_noalloc: the call needs more scratch than its static array */
} bgb_status;

typedef enum { BGB_F32 = 0, BGB_F16 = 1, BGB_BF16 = 2 } bgb_dtype;

typedef enum { BGB_MODE_FBI = 0, BGB_MODE_BITNET = 1, BGB_MODE_TERNARY = 2 } bgb_mode;

typedef enum {
    BGB_OP_PACK_FBI = 0,
    BGB_OP_PACK_BITNET = 1,
    BGB_OP_FBI_LINEAR = 2,
    BGB_OP_BITLINEAR = 3,
    BGB_OP_BITLINEAR158 = 4,
    BGB_OP_FBI_BACKWARD = 5
} bgb_op;

/* Integer conversion of the clipped quantizer input v_c (eq. (4) gives none):
 * truncation toward zero (the default; it keeps |q| <= Q_b - 1 through the
 * clip margin) or round to nearest, ties to even, then clamp to +-(Q_b - 1). */
typedef enum { BGB_ROUND_TRUNC = 0, BGB_ROUND_RNE = 1 } bgb_round_mode;

/* What gamma = ||LN(x)||_inf is taken over: the whole M x K input (the
 * default; section 一 speaks of the input matrix's maximum) or each token. */
typedef enum { BGB_GAMMA_TENSOR = 0, BGB_GAMMA_TOKEN = 1 } bgb_gamma_scope;

/* The codes' range: symmetric (eq. (4), the default) or non-negative (eq. (6),
 * for activations ahead of a non-linear function): Clip((h - eta) Q_b / gamma,
 * eps, Q_b - eps) with eta = min h over gamma's scope and gamma = ||h||_inf as
 * eq. (5) defines it, codes in [0, Q_b - 1]. The page gives eq. (7) only, so
 * the output is W~ q beta gamma / Q_b for both ranges (eta is not added back). */
typedef enum { BGB_RANGE_SYMMETRIC = 0, BGB_RANGE_NONNEG = 1 } bgb_act_range;

/* Activation quantization parameters of BitLinear ("BitNet b1.58: 1bit LLM时代",
 * section 一, eq. (4)-(6), (8)). */
typedef struct {
    double ln_eps;   /* LayerNorm epsilon added to the variance, > 0 (1e-5) */
    int bits;        /* b in Q_b = 2^(b-1); 2..8 (8 -> Q_b = 128, int8 codes) */
    float q_eps;     /* clip margin in (0, 1): codes are clipped to [-Q_b+eps, Q_b-eps] (1e-3) */
    int round_mode;  /* bgb_round_mode (BGB_ROUND_TRUNC) */
    int gamma_scope; /* bgb_gamma_scope (BGB_GAMMA_TENSOR) */
    int act_range;   /* bgb_act_range (BGB_RANGE_SYMMETRIC) */
} bgb_quant_params;

/* Size in bytes of the packed array P for a K x N weight (0 if K is invalid). */
size_t bgb_packed_bytes(int64_t K, int64_t N);

/* Workspace bytes that `op` needs for these sizes (M is ignored by the packs). */
size_t bgb_workspace_bytes(int op, int64_t M, int64_t K, int64_t N);

/*
 * binarize_pack -- one-time weight conversion.
 *
 * mode BGB_MODE_FBI (FBI-linear paragraph of the FBI-LLM news rewrite; tie
 * rule from the BitNet blog, eq. (2)): s_ij = +1 iff W_ij > 0, else -1
 * (zeros and NaN give -1; positive subnormals give +1).
 *   alpha_j = mean_i |W_ij| over the K inputs of output column j, summed in
 *   fp64 and rounded once to fp32 (then to fp16 by round-to-nearest-even
 *   when alpha_dtype == BGB_F16). alpha: [N] of alpha_dtype (F32 or F16).
 *   beta and centre are ignored (may be NULL).
 * mode BGB_MODE_BITNET (BitNet blog, eq. (1)-(3) and (8)):
 *   centre c = mean(W), beta = ||W||_1/(K N), each an fp64 sum rounded once to
 *   fp32 and written to device scalars `centre` and `beta`;
 *   s_ij = +1 iff W_ij > c (compared exactly in fp32), else -1.
 *   alpha/alpha_dtype are ignored (may be NULL).
 * mode BGB_MODE_TERNARY (BitNet b1.58, same blog, section 二, eq. (9)-(11)):
 *   gamma_w = mean |W| (fp64 sum rounded once to fp32), written to `beta`
 *   (it is the beta of eq. (8) for these weights); t_ij = RoundClip(
 *   W_ij / (gamma_w + 1e-5), -1, 1), the divisor and quotient in fp32 and
 *   round() to nearest even. P holds two planes of the binary format, each
 *   bgb_packed_bytes(K, N) bytes: bit 1 in the first iff t_ij = +1, in the
 *   second iff t_ij = -1. `centre` (mean W) is written when not NULL.
 * W: [K][N] float32 (input). P: bgb_packed_bytes(K, N) bytes (output; twice
 * that for BGB_MODE_TERNARY).
 * ws: bgb_workspace_bytes(BGB_OP_PACK_FBI or _BITNET, 0, K, N) bytes (the
 * ternary mode uses the BITNET size).
 * Errors: BGB_EINVAL (null, K % 32 != 0, sizes, alignment, workspace),
 *         BGB_EUNSUPPORTED (alpha dtype not F32/F16, unknown mode), BGB_EHIP.
 */
int binarize_pack(const float* W, int64_t K, int64_t N, int mode, uint32_t* P,
                  void* alpha, int alpha_dtype, float* beta, float* centre,
                  void* ws, size_t ws_bytes, void* stream);

/*
 * fbi_linear_w1a16 -- FBI-linear forward (W1A16).
 *   y[m][j] = alpha_j * sum_i s_ij * x[m][i]
 * x: [M][K] bf16 or f16 (x_dtype BGB_BF16 / BGB_F16). P: packed signs (above).
 * alpha: [N] in alpha_dtype (F32 or F16), used as given (a trained scale is
 * accepted). y: [M][N] in y_dtype (F32, BF16 or F16; 16-bit outputs are
 * rounded to nearest even). Products of +-1 and x are exact; sums use fp32
 * accumulation on the matrix cores; alpha is applied once to the fp32 sum.
 * M <= 64 runs the decode kernels (activations staged in LDS), M > 64 the
 * MFMA GEMM. One token with K <= 16384 runs on the fp8 matrix cores: the token,
 * scaled by a power of two into [8, 16), as five integer limbs of quantum
 * 2^-16, whose column sums are exact; each activation is then carried to
 * within max|x| 2^-20 (exactly for values within about 2^-12 of the largest
 * magnitude, and for integers while the largest magnitude is below 2^20), and
 * a token holding an inf or a NaN gives NaN outputs.
 * ws: bgb_workspace_bytes(BGB_OP_FBI_LINEAR, M, K, N) bytes. When that is 0
 * (one token with K <= 16384, up to 16 tokens whose activations fit on chip
 * whole, and decode shapes whose K range is not split) ws is neither read nor
 * written and may be NULL. Decode shapes whose K range is split over several
 * blocks keep fp32 partial sums there ([splits][M][N]), added in a fixed
 * order by a second launch; likewise the GEMM for shapes whose K range it
 * splits (fp32 partial sums [splits][M][N]). The GEMM reads x in place.
 * Errors: BGB_EINVAL, BGB_EUNSUPPORTED (dtypes), BGB_EHIP.
 */
int fbi_linear_w1a16(const void* x, int x_dtype, int64_t M, int64_t K, int64_t N,
                     const uint32_t* P, const void* alpha, int alpha_dtype,
                     void* y, int y_dtype, void* ws, size_t ws_bytes, void* stream);

/* One FBI-linear of a group: its activations, packed signs, scales, output
 * and shape, with the layouts of fbi_linear_w1a16. */
typedef struct {
    const void* x;        /* [M][K] 16-bit */
    const uint32_t* P;    /* packed signs of the K x N weight */
    const void* alpha;    /* [N] */
    void* y;              /* [M][N] */
    int64_t K, N;
} bgb_w1a16_item;

#define BGB_GROUP_MAX 8

/*
 * fbi_linear_w1a16_group -- several independent FBI-linears (FBI-linear
 * paragraph of the FBI-LLM news rewrite; the model replaces every linear of a
 * layer) over the same number of tokens M and the same dtypes: for each item,
 * the result of fbi_linear_w1a16(item.x, x_dtype, M, item.K, item.N, item.P,
 * item.alpha, alpha_dtype, item.y, y_dtype, ...). All items run in one
 * launch (each item split into column groups of its own, one per block) for a
 * single token (M = 1) with every K <= 12928, for 2 <= M <= 16 tokens
 * when every item's tokens fit in LDS (about 140 KB for M (K + 136) 16-bit
 * values), and for 17 <= M <= 64 tokens (each item as 64-token x 256-column
 * matrix-core tiles, its K range split into equal parts whose fp32 sums one
 * reduce launch for the whole group adds in part order). Up to 16 tokens,
 * when some items do not fit those limits, the others (if at least two) run
 * as one launch and the rest one after another in the order given; beyond
 * that, all run one after another. Sums are accumulated in fp32 in a fixed order,
 * so results are the same from run to run; the one-launch form may group a
 * linear's K range differently from fbi_linear_w1a16 (a different rounding
 * order of the fp32 sum, not bit-identical to it).
 * items: a host array of `count` items (0 <= count <= BGB_GROUP_MAX), read
 * during the call only. Items with N = 0 are skipped; every other item is
 * checked as fbi_linear_w1a16 checks its arguments. No output may overlap
 * any item's x, P, alpha or another item's y (the items may run
 * concurrently): BGB_EINVAL otherwise.
 * ws: bgb_group_workspace_bytes(items, count, M) bytes (0 for the one- and
 * few-token one-launch forms, where ws may be NULL; for 17 <= M <= 64 the
 * parts' raw sums).
 * Errors: BGB_EINVAL, BGB_EUNSUPPORTED (dtypes), BGB_EHIP; a rejected call
 * launches nothing.
 */
int fbi_linear_w1a16_group(const bgb_w1a16_item* items, int count, int64_t M, int x_dtype,
                           int alpha_dtype, int y_dtype, void* ws, size_t ws_bytes,
                           void* stream);

/* Workspace bytes of fbi_linear_w1a16_group for these items (the largest
 * item's fbi_linear_w1a16 workspace, 0 for the one-launch form). */
size_t bgb_group_workspace_bytes(const bgb_w1a16_item* items, int count, int64_t M);

/*
 * fbi_pack_transposed -- the signs of S^T for the backward product (FBI-LLM
 * news rewrite, training paragraph: gradients pass the sign function by the
 * straight-through estimator, so dX needs the same signs transposed).
 * P: the packed signs of a K x N weight (binarize_pack, FBI mode). PT
 * (output): the packed format of the 2N x K matrix [S^T; S^T] (the
 * transposed signs twice along the contraction axis),
 * bgb_packed_bytes(2 N, K) bytes, 16-byte aligned. N % 32 == 0.
 * Errors: BGB_EINVAL (null, sizes, alignment), BGB_EHIP.
 */
int fbi_pack_transposed(const uint32_t* P, int64_t K, int64_t N, uint32_t* PT, void* stream);

/*
 * fbi_linear_w1a16_backward -- FBI-linear backward through the identity
 * straight-through estimator (the pages state no clipping):
 *   dX[m][i] = sum_j s_ij alpha_j dY[m][j]            [M][K], dx_dtype
 *   dalpha_j = sum_m dY[m][j] sum_i s_ij x[m][i]      [N] fp32
 *   dW[i][j] = alpha_j sum_m x[m][i] dY[m][j]         [K][N] fp32
 * (dW is the gradient of W_b = alpha * sign(W) passed to the latent W.)
 * dy: [M][N], x: [M][K], both of `dtype` (BF16 or F16). Any of dx, dalpha,
 * dw may be NULL (not computed); dx needs PT (fbi_pack_transposed), dalpha
 * needs x and P, dw needs x. N % 32 == 0. When dx is requested, 2 N K < 2^31
 * as well (dX runs the forward product over the 2N x K operand [S^T; S^T]).
 * Numerics: dX runs the forward product on g = fl32(alpha_j dY) carried as
 * two bf16 halves (g_hi + g_lo, about 16 significant bits), fp32
 * accumulation; dalpha is the forward at alpha = 1 (fp32 sums) times dY,
 * summed over tokens in fp64 in token order; dW is a 16-bit matrix-core
 * product over the tokens with fp32 accumulation, times alpha_j in fp32.
 * ws: bgb_workspace_bytes(BGB_OP_FBI_BACKWARD, M, K, N) bytes.
 * Errors: BGB_EINVAL, BGB_EUNSUPPORTED (dtypes), BGB_EHIP.
 */
int fbi_linear_w1a16_backward(const void* dy, const void* x, int dtype, int64_t M, int64_t K, int64_t N,
                              const uint32_t* P, const uint32_t* PT, const void* alpha, int alpha_dtype,
                              void* dx, int dx_dtype, float* dalpha, float* dw, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * bitlinear_w1a8 -- BitLinear forward (BitNet blog, section 一, eq. (4)-(8)).
 *   h = LN(x) per token (biased variance, no affine): E(x), Var(x) in fp64,
 *       then h = fl32(fl32(x - fl32(E)) * fl32(1/sqrt(Var + ln_eps)))
 *   gamma = max |h| over the whole M x K tensor (qp->gamma_scope TENSOR),
 *       or gamma_m = max_i |h[m][i]| per token (TOKEN)
 *   q = trunc(clip(fl32(h * Q_b / gamma), -(Q_b - q_eps), Q_b - q_eps))
 *       (qp->round_mode TRUNC; RNE rounds to nearest even instead and
 *       clamps to +-(Q_b - 1)); q = 0 when gamma == 0; |q| <= Q_b - 1
 *   acc[m][j] = sum_i s_ij * q[m][i]           (exact int32)
 *   y[m][j] = fl32(float(acc) * fl32(fl32(beta * gamma) / Q_b))
 *       (gamma_m of the row's token for the TOKEN scope)
 * x: [M][K] F32 or BF16. P: packed signs of W - c (binarize_pack BITNET).
 * beta: device scalar from binarize_pack. qp: host pointer (NULL = defaults
 * ln_eps 1e-5, bits 8, q_eps 1e-3, TRUNC, TENSOR). y: [M][N] float32.
 * Optional outputs (NULL to skip): xq_opt int8 [M][K] codes, gamma_opt device
 * float [1] (TENSOR) or [M] (TOKEN), acc_opt int32 [M][N].
 * ws: bgb_workspace_bytes(BGB_OP_BITLINEAR, M, K, N) bytes.
 * M <= 32 runs the memory-bound decode kernels, M > 32 the int8 MFMA GEMM.
 * Errors: BGB_EINVAL, BGB_EUNSUPPORTED, BGB_EHIP.
 */
int bitlinear_w1a8(const void* x, int x_dtype, int64_t M, int64_t K, int64_t N,
                   const uint32_t* P, const float* beta, const bgb_quant_params* qp,
                   float* y, int8_t* xq_opt, float* gamma_opt, int32_t* acc_opt,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * bitlinear_w1a8_noalloc -- bitlinear_w1a8 for callers that cannot allocate
 * device memory or hand over a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. Same arguments, results and
 * kernels as bitlinear_w1a8, minus (ws, ws_bytes): the workspace is a static
 * device array of BGB_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 * held from the library's load until the process ends. The call allocates
 * nothing; its first call on a device looks the array's address up once.
 * Calls that overlap on one GPU (concurrent streams, or host threads) share
 * that array and race: order them, or use bitlinear_w1a8 with workspaces of
 * their own. No call relies on what a previous one left in the array.
 * Errors: as bitlinear_w1a8, and BGB_ESCRATCH (nothing launched) when
 * bgb_workspace_bytes(BGB_OP_BITLINEAR, M, K, N) exceeds
 * BGB_NOALLOC_SCRATCH_BYTES (e.g. 2048 tokens x 4096 features need 8.1 MiB,
 * 4096 x 4096 need 16.1 MiB; calls whose launch plan splits K also hold their
 * partial sums there).
 */
#define BGB_NOALLOC_SCRATCH_BYTES (64u << 20)
size_t bgb_noalloc_scratch_bytes(void);
int bitlinear_w1a8_noalloc(const void* x, int x_dtype, int64_t M, int64_t K, int64_t N,
                           const uint32_t* P, const float* beta, const bgb_quant_params* qp,
                           float* y, int8_t* xq_opt, float* gamma_opt, int32_t* acc_opt,
                           void* stream);

/*
 * bitlinear_quantize + bitlinear_matmul -- the two stages of bitlinear_w1a8,
 * for callers that apply several BitLinear weights to one input (the
 * q/k/v or gate/up projections of a block share theirs).
 * bitlinear_quantize runs the prologue (LN, gamma, codes) for x [M][K] and
 * leaves the codes, their row sums and gamma in `ws` (sized by
 * bgb_workspace_bytes(BGB_OP_BITLINEAR, M, K, N) for the largest N used);
 * xq_opt / gamma_opt are optional copies as above.
 * bitlinear_matmul then computes y (and optionally acc) for one packed weight
 * from that workspace; M, K, qp->bits and qp->gamma_scope must match the
 * quantize call, and
 * the two calls must be ordered on one stream. bitlinear_w1a8 is exactly
 * bitlinear_quantize followed by bitlinear_matmul.
 */
int bitlinear_quantize(const void* x, int x_dtype, int64_t M, int64_t K,
                       const bgb_quant_params* qp, int8_t* xq_opt, float* gamma_opt,
                       void* ws, size_t ws_bytes, void* stream);
int bitlinear_matmul(int64_t M, int64_t K, int64_t N, const uint32_t* P, const float* beta,
                     const bgb_quant_params* qp, float* y, int32_t* acc_opt,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * bitlinear158_w1a8 + bitlinear158_matmul -- BitNet b1.58 forward: ternary
 * weights with 8-bit activations ("BitNet b1.58: 1bit LLM时代", section 二:
 * weights by eq. (9)-(11); activations quantized as in section 一, which
 * section 二 keeps).
 *   h, gamma, q: exactly as bitlinear_w1a8 (same qp options)
 *   acc[m][j] = sum_i t_ij * q[m][i], t in {-1, 0, 1}      (exact int32)
 *   y[m][j] = fl32(float(acc) * fl32(fl32(beta * gamma) / Q_b))
 * P: the two planes from binarize_pack(BGB_MODE_TERNARY) (2 x
 * bgb_packed_bytes(K, N) bytes); beta: its gamma_w = mean |W|, which is the
 * beta of eq. (8) for the weights. ws: bgb_workspace_bytes(
 * BGB_OP_BITLINEAR158, M, K, N) bytes. Everything else (taps, errors, the M
 * dispatch, pairing with bitlinear_quantize) is as for the binary weights.
 */
int bitlinear158_w1a8(const void* x, int x_dtype, int64_t M, int64_t K, int64_t N,
                      const uint32_t* P, const float* beta, const bgb_quant_params* qp,
                      float* y, int8_t* xq_opt, float* gamma_opt, int32_t* acc_opt,
                      void* ws, size_t ws_bytes, void* stream);
int bitlinear158_matmul(int64_t M, int64_t K, int64_t N, const uint32_t* P, const float* beta,
                        const bgb_quant_params* qp, float* y, int32_t* acc_opt,
                        void* ws, size_t ws_bytes, void* stream);

/* Message for a status code (static string). */
const char* bgb_status_string(int status);

/* The hipError_t value behind the most recent BGB_EHIP (0 if none). */
int bgb_last_hip_error(void);

/* Library version string. */
const char* bgb_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BGB_H */
