// Internal declarations shared by the C-ABI layer and the kernel files.
// Host-side only: launcher prototypes, workspace layout, size rules.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bgb {

constexpr int kWords4 = 4;             // words per 16-byte column tile (128 rows)
constexpr int kGemvMaxM = 32;          // W1A8: M <= 32 -> decode (streaming) kernels, above: MFMA GEMM
constexpr int kW1A16DecodeMaxM = 64;   // W1A16: M <= 64 -> decode kernels, above: MFMA GEMM
constexpr int kSmallPrologueM = 16;    // M <= 16 -> single-block LN + quant prologue
constexpr int kMaxK = 524288;

inline int64_t words_per_col(int64_t K) { return K / 32; }                // T
inline int64_t tiles_per_col(int64_t K) { return (K / 32 + 3) / 4; }      // TQ
inline int64_t padded_k(int64_t K) { return tiles_per_col(K) * 128; }    // Kp

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// ---- workspace layouts (all offsets 256-byte aligned) -----------------------
struct PackFbiWs {          // fp64 partial |W| sums per (tile, column)
    size_t colsum, total;
    static PackFbiWs make(int64_t K, int64_t N) {
        PackFbiWs w{};
        w.colsum = 0;
        w.total = align256(size_t(tiles_per_col(K)) * size_t(N) * sizeof(double));
        return w;
    }
};

constexpr int kBitnetReduceBlocks = 1024;
struct PackBitnetWs {       // fp64 (sum W, sum |W|) per reduction block, then a float scratch (mean W
    size_t partial, scratch, total;   //  when the caller does not ask for it)
    static PackBitnetWs make() {
        PackBitnetWs w{};
        w.partial = 0;
        w.scratch = align256(size_t(kBitnetReduceBlocks) * 2 * sizeof(double));
        w.total = w.scratch + 256;
        return w;
    }
};

// BitNet b1.58 weights: RoundClip(W / (mean|W| + eps), -1, 1) with this eps.
constexpr float kTernaryEps = 1e-5f;

// GEMM launch plan (a pure function of the shape): token fragments per wave
// (BM = 16 nn), K splits and stages per split, tile grid.
struct GemmPlan {
    int nn, nw, splits, per, T, ntm, ntj;   // nw waves of 64 columns per block
};
GemmPlan gemm_plan(int64_t M, int64_t K, int64_t N, bool w1a8, bool tern);
size_t gemm_partial_bytes(int64_t M, int64_t K, int64_t N, bool w1a8, bool tern);   // [splits][M][N] x 4 B, or 0

// Chunked W1A16 decode plan (a pure function of the shape): tokens per block
// 16 tf, tiles per wave and chunk tpw, fragments per block fb, K splits (each
// split takes cps chunks; splits > 1 store raw sums, then a reduce pass).
struct DecodekPlan {
    int tf, tpw, fb, splits, cps, nchunks;
};
DecodekPlan decodek_plan(int64_t M, int64_t K, int64_t N);
// Which W1A16 decode kernel serves M <= kW1A16DecodeMaxM, and its workspace
// (raw split sums, [splits][M][N] fp32; 0 when nothing is split).
size_t w1a16_decode_ws_bytes(int64_t M, int64_t K, int64_t N);

struct FbiLinearWs {        // split-K partial sums (decode or GEMM), when the plan splits K
    size_t part, total;
    static FbiLinearWs make(int64_t M, int64_t K, int64_t N) {
        FbiLinearWs w{};
        w.part = 0;
        w.total = M <= kW1A16DecodeMaxM ? w1a16_decode_ws_bytes(M, K, N) : gemm_partial_bytes(M, K, N, false, false);
        return w;
    }
};

// FBI-linear backward: the split scaled gradient [M][2N] bf16, z [M][N] fp32,
// the fp64 chunk sums of dalpha, a vector of ones (max(K, N) fp32), then the
// forward calls' own workspace.
size_t dalpha_part_bytes(int64_t M, int64_t N);
struct FbiBackwardWs {
    size_t g2, z, part, ones, inner, total;
    static FbiBackwardWs make(int64_t M, int64_t K, int64_t N) {
        FbiBackwardWs w{};
        w.g2 = 0;
        w.z = align256(size_t(M) * size_t(2 * N) * 2);
        w.part = w.z + align256(size_t(M) * size_t(N) * 4);
        w.ones = w.part + align256(dalpha_part_bytes(M, N));
        w.inner = w.ones + align256(size_t(K > N ? K : N) * 4);
        const size_t a = FbiLinearWs::make(M, 2 * N, K).total, b = FbiLinearWs::make(M, K, N).total;
        w.total = w.inner + align256(a > b ? a : b);
        return w;
    }
};

struct BitlinearWs {
    size_t stats, gamma, rowsum, q, mins, part, total;
    // N = 0: the prologue's regions only (what bitlinear_quantize touches)
    // tern: ternary weights (their GEMM plan, hence split partials, differ)
    static BitlinearWs make(int64_t M, int64_t K, int64_t N, bool tern = false) {
        BitlinearWs w{};
        w.stats = 0;                                               // float [M][3] mu32, rstd32, rowmax
        w.gamma = w.stats + align256((size_t(M) * 3 + size_t(M + 3) / 4) * sizeof(float));  // + block maxima
        w.rowsum = w.gamma + 256;                                  // int32 [M]
        w.q = w.rowsum + align256(size_t(M) * sizeof(int32_t));    // int8 [M][Kp], layout per path
        w.mins = w.q + align256(size_t(M) * size_t(padded_k(K)));  // float [M] + block minima (eq. (6) range)
        w.part = w.mins + align256((size_t(M) + size_t(M + 3) / 4) * sizeof(float));   // int32 split-K partials
        w.total = w.part + (M > kGemvMaxM && N > 0 ? gemm_partial_bytes(M, K, N, true, tern) : 0);
        return w;
    }
};

// Record a HIP error for bgb_last_hip_error() (entry points outside abi.hip).
void set_last_hip_error(int e);

// ---- launchers (each returns hipGetLastError() after its launches) -----------
hipError_t launch_pack(const float* W, int64_t K, int64_t N, int mode, uint32_t* P,
                       void* alpha, int alpha_f16, float* beta, float* centre,
                       void* ws, hipStream_t s);

// q layout written by the prologue: 0 = decode kernel layout, 1 = GEMM layout
// mins != NULL: the non-negative range of eq. (6) (row minima [M] and block
// minima there; lo = fl32(q_eps) is the lower clip)
hipError_t launch_ln_quant(const void* x, int x_bf16, int64_t M, int64_t K, double ln_eps,
                           float qb, float lim, int rne, int token, float* mins, float lo, int layout,
                           int8_t* q, int32_t* rowsum, float* stats, float* gamma_ws, int8_t* xq_opt,
                           float* gamma_opt, hipStream_t s);

hipError_t launch_w1a16_gemm(const uint16_t* x, int x_f16, int64_t M, int64_t K, int64_t N,
                             const uint32_t* P, const void* alpha, int alpha_f16, void* y,
                             int y_dtype, void* part, hipStream_t s);

hipError_t launch_w1a8_gemv(const int8_t* q, const int32_t* rowsum, const float* gamma,
                            int gstride, const float* beta, float qb, int64_t M, int64_t K,
                            int64_t N, const uint32_t* P, float* y, int32_t* acc_opt, int tern,
                            hipStream_t s);

// Single-token fused kernels (prologue / activation staging inside the GEMV).
bool w1a8_decode1_supported(int64_t K);
hipError_t launch_w1a8_decode1(const void* x, int x_bf16, int64_t K, int64_t N, double eps, float qb, float lim,
                               int rne, const uint32_t* P, const float* beta, float* y, int32_t* acc_opt,
                               int8_t* xq_opt, float* gamma_opt, int tern, hipStream_t s);
bool w1a16_decode1_supported(int64_t K);
// 2 <= M <= 16 tokens staged in LDS by every block (M (Kp + 8) 2 bytes <= 140 KB)
bool w1a16_decodem_supported(int64_t M, int64_t K);
// 1 <= M <= 64 tokens, K staged in chunks (any K)
bool w1a16_decodek_supported(int64_t M, int64_t K);
hipError_t launch_w1a16_decodek(const void* x, int x_f16, int64_t M, int64_t K, int64_t N, const uint32_t* P,
                                const void* alpha, int alpha_f16, void* y, int y_dtype, float* part,
                                hipStream_t s);
// y[m][j] = alpha_j * sum_z part[z][m][j], z in order (gemm.hip)
hipError_t launch_w1a16_splitk_reduce(const float* part, int splits, int64_t M, int64_t N, const void* alpha,
                                      int alpha_f16, void* y, int y_dtype, hipStream_t s);
hipError_t launch_w1a16_decodem(const void* x, int x_f16, int64_t M, int64_t K, int64_t N, const uint32_t* P,
                                const void* alpha, int alpha_f16, void* y, int y_dtype, hipStream_t s);
hipError_t launch_w1a16_decode1(const void* x, int x_f16, int64_t K, int64_t N, const uint32_t* P,
                                const void* alpha, int alpha_f16, void* y, int y_dtype, hipStream_t s);
// Several independent single-token linears (at most kGroupMax, each with
// w1a16_decode1_supported(K)) in one launch; empty ones (N = 0) are skipped.
constexpr int kGroupMax = 8;
struct W1a16Item {
    const void* x;
    const uint32_t* P;
    const void* alpha;
    void* y;
    int64_t K, N;
};
bool w1a16_decode1_group_item_ok(int64_t K);
bool w1a16_decode1_group_supported(const W1a16Item* items, int count);
hipError_t launch_w1a16_decode1_group(const W1a16Item* items, int count, int x_f16, int alpha_f16, int y_dtype,
                                      hipStream_t s);
// 17 <= M <= 64 tokens: the MFMA GEMM tile per item in one launch, K split
// per item, the parts' raw sums (workspace, w1a16_gemm_group_ws_bytes) added
// in part order by one reduce launch for the whole group.
bool w1a16_gemm_group_supported(const W1a16Item* items, int count, int64_t M);
size_t w1a16_gemm_group_ws_bytes(const W1a16Item* items, int count, int64_t M);
hipError_t launch_w1a16_gemm_group(const W1a16Item* items, int count, int64_t M, int x_f16, int alpha_f16,
                                   int y_dtype, void* ws, hipStream_t s);
// 2 <= M <= 16 tokens, every item's tokens staged whole in LDS
// (w1a16_decodem_supported), one launch.
bool w1a16_decodem_group_supported(const W1a16Item* items, int count, int64_t M);
hipError_t launch_w1a16_decodem_group(const W1a16Item* items, int count, int64_t M, int x_f16, int alpha_f16,
                                      int y_dtype, hipStream_t s);

// FBI-linear backward pieces (backward.hip).
hipError_t launch_pack_transpose(const uint32_t* P, int64_t K, int64_t N, uint32_t* PT, hipStream_t s);
hipError_t launch_fbi_backward_parts(const void* dy, int dy_f16, const void* x, int64_t M, int64_t K, int64_t N,
                                     const void* alpha, int alpha_f16, uint16_t* g2, float* ones, int64_t nones,
                                     float* dw, hipStream_t s);
hipError_t launch_dalpha(const void* dy, int dy_f16, const float* z, int64_t M, int64_t N, double* part,
                         float* dalpha, hipStream_t s);
size_t dalpha_part_bytes(int64_t M, int64_t N);     // fp64 chunk sums [chunks][N]

hipError_t launch_w1a8_gemm(const int8_t* q, const int32_t* rowsum, const float* gamma,
                            int gstride, const float* beta, float qb, int64_t M, int64_t K,
                            int64_t N, const uint32_t* P, float* y, int32_t* acc_opt, void* part,
                            int tern, hipStream_t s);

}  // namespace bgb
