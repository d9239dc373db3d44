// Prefill kernels: a dense contraction, so it runs on the matrix cores.
// FBI-linear W1A16 (FBI-LLM news rewrite, FBI-linear paragraph) on bf16/f16
// MFMA with fp32 accumulation; BitLinear W1A8 ("BitNet b1.58: 1bit LLM时代",
// section 一, eq. (7)) on int8 MFMA with int32 accumulation.
//
// Tiling: a block of 4 waves computes a 256-column x BM-token tile (BM = 128
// or 64); wave w owns columns 64w..64w+63 (four 16-column MFMA fragments)
// for all BM tokens (NN = BM/16 token fragments): 4 x NN accumulators of
// 16x16. A launch may split the K range over gridDim.y blocks per tile; each
// split then stores its raw sums and a second kernel adds the splits in a
// fixed order (so results are identical from run to run) and applies the
// epilogue.
//
// Pipeline: the K loop runs over stages of 128 bytes of activations per token
// (64 rows of bf16/f16, 128 rows of int8). Activation stages go from global
// memory straight into LDS with global_load_lds_dwordx4 (no VGPR staging),
// four stages in flight in a ring of four buffers; the block's 4 KB sign tile
// of a stage goes the same way into a second ring. One s_waitcnt + s_barrier
// per stage; the waits are explicit because only the kernel knows how many
// DMA operations a stage issues.
//
// LDS layout of a stage: token row t at t*128 bytes, its eight 16-byte chunks
// XOR-swizzled by a function of bits 1..3 of t, so that the 16-byte B-operand
// reads of every 16 consecutive lanes hit 16 distinct 16-byte bank groups of
// 256 bytes, and those of every 32 lanes 32 distinct groups of 512 bytes (a
// swizzle on bits 2..3 alone left two-way conflicts within 16 lanes:
// SQ_LDS_BANK_CONFLICT read half of SQ_LDS_IDX_ACTIVE). The DMA writes lane L
// of an instruction to chunk base+L, so the swizzle is applied by choosing the
// source chunk per lane.
//
// Sign decoding (A operand, rows = output columns), per MFMA:
// * W1A16: lane group g takes word g>>1 of the stage and, for MFMA half v,
//   its 16-byte chunk u = 2v + (g&1): rows 8u..8u+7 in their natural order,
//   dword e holding rows 8u+2e and 8u+2e+1. The lane's half of the sign
//   word is regrouped once per stage (gather_pairs: the two rows of each
//   pair 16 bits apart), so that one bitop3 of the shifted word gives both
//   sign bits of dword e over the bit pattern of 1.0. The activations are
//   read from x itself, no reordered copy.
// * W1A8: lane group g takes word g, MFMA v = 0..1, dword d carries rows
//   4v+d+8e (byte e) as 0/1 bytes; sum s q = 2 sum b q - sum q with the row
//   sums of the codes from the prologue, which writes the codes in this order.
#include "bgb_device.hpp"
#include "bgb_internal.hpp"

#include <type_traits>

namespace bgb {

constexpr int kRing = 4;            // stages in the LDS rings

template <bool kF16>
BGB_DEV f32x4_t mfma16g(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
    if constexpr (kF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// s_waitcnt vmcnt(N) leaving the LDS/export counters alone (gfx9 encoding).
template <int N>
BGB_DEV void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// s_waitcnt vmcnt(N) lgkmcnt(0).
template <int N>
BGB_DEV void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

BGB_DEV void dma16(const void* src, uint8_t* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 0);
}

// Chunk swizzles of a stage row (see the header comment): XOR masks in 0..7
// from bits 1..3 of the token row. Over the 8 rows of one parity each takes
// all 8 values (16-lane passes); over the 4 rows of one residue mod 4 each
// takes one value from each coset of the chunk pair a half-wave reads ({c,
// c^2} for W1A8, {c, c^1} for W1A16: 32-lane passes).
BGB_DEV int swz16(int t) { return (2 * ((t >> 2) & 3)) | ((t >> 1) & 1); }
BGB_DEV int swz8(int t) { return (((t >> 2) & 1) | (((t >> 3) & 1) << 2)) ^ (t & 2); }

// The sign bits a W1A16 lane needs from a 32-row word w, placed for the
// decode: with sel picking bytes (h, h + 2, h, h + 2) of w (rows 8h..8h+7 and
// 16+8h..16+8h+7), the result holds the even rows of byte h at bits 0..3,
// those of byte h + 2 at bits 8..11, and the odd rows of the two bytes at
// bits 16..19 and 24..27 -- so rows 2i and 2i + 1 of a chunk sit 16 bits
// apart. One byte permute, then two halving steps compress each byte's
// even (low half) or odd (high half) bits into its low nibble.
BGB_DEV uint32_t gather_pairs(uint32_t w, uint32_t sel) {
    const uint32_t z = __builtin_amdgcn_perm(w, w, sel);
    uint32_t m = ((z & 0x0000FFFFu) | ((z >> 1) & 0xFFFF0000u)) & 0x55555555u;
    m = (m | (m >> 1)) & 0x33333333u;
    return (m | (m >> 2)) & 0x0F0F0F0Fu;
}

// 16 zero bytes in global memory: the DMA source for activation chunks past K.
__device__ __attribute__((aligned(16))) uint32_t g_zero16[4];

// ------------------------------------------------------------------- plan ----
// Cost model, in microseconds: a stage of a 128-token block (two blocks per
// CU sharing the matrix cores) takes kStageUs, a 64-token one kStageUs * 0.6;
// each block adds kFixedStages stages of pipeline fill and epilogue; a split
// launch adds the reduce pass (its traffic at kReduceBytesPerUs plus one
// launch).
namespace {
constexpr double kStageUs = 1.6;
constexpr double kFixedStages = 3.0;
constexpr double kReduceBytesPerUs = 5.0e6;
constexpr double kLaunchUs = 2.0;
constexpr int kSlots = 512;         // resident blocks: 2 per CU on 256 CUs
}  // namespace

GemmPlan gemm_plan(int64_t M, int64_t K, int64_t N, bool w1a8, bool tern) {
    const int T = int(w1a8 ? tiles_per_col(K) : 2 * tiles_per_col(K));
    const int ntj = int((N + 255) / 256);
    GemmPlan best{};
    best.nw = 4;
    double best_t = 1e300;
    for (int nn : {8, 4}) {
        if (tern && nn == 8) continue;     // ternary: two accumulator sets, 64-token tiles only
        const int ntm = int((M + 16 * nn - 1) / (16 * nn));
        const int64_t tiles = int64_t(ntm) * ntj;
        const double stage = nn == 8 ? 1.0 : 0.6;
        for (int S : {1, 2, 3, 4, 6, 8, 12, 16, 24, 32}) {
            const int per = (T + S - 1) / S;
            const int splits = (T + per - 1) / per;
            if (splits != S) continue;                       // no S-way split with equal ranges
            if (S > 1 && per < 2) break;
            const int64_t units = tiles * splits;
            const double rounds = double((units + kSlots - 1) / kSlots);
            double t = rounds * (per + kFixedStages) * stage * kStageUs;
            if (splits > 1) t += (double(splits + 1) * double(M) * double(N) * 4.0) / kReduceBytesPerUs + kLaunchUs;
            if (t < best_t) {
                best_t = t;
                best.nn = nn;
                best.splits = splits;
                best.per = per;
                best.T = T;
                best.ntm = ntm;
                best.ntj = ntj;
            }
        }
    }
    return best;
}

size_t gemm_partial_bytes(int64_t M, int64_t K, int64_t N, bool w1a8, bool tern) {
    const GemmPlan p = gemm_plan(M, K, N, w1a8, tern);
    return p.splits > 1 ? align256(size_t(p.splits) * size_t(M) * size_t(N) * 4) : 0;
}

// ------------------------------------------------------------------ kernel ----
struct GemmArgs {
    const uint8_t* act;        // x (W1A16, [M][K] 16-bit) or q (W1A8, [M][Kp] int8)
    int64_t row_bytes;
    int64_t K;
    const uint32_t* P;
    int64_t M, N;
    int T, per, ntj, ntiles;
    // W1A16 epilogue
    const void* alpha;
    int alpha_f16;
    void* y;
    int y_dtype;
    // W1A8 epilogue
    const int32_t* rowsum;
    const float* gamma;        // gamma of token m at gamma[m * gstride] (gstride 0: one for the tensor)
    int gstride;
    const float* beta;
    float qb;
    int32_t* acc_opt;
    int tern;                  // ternary weights: the raw sum is already sum t q (no 2 s - rowsum)
    // raw sums per split when the K range is split: [splits][M][N]
    void* part;
};

BGB_DEV float alpha_at(const void* alpha, int alpha_f16, int64_t j) {
    return alpha_f16 ? f16_to_f32(static_cast<const uint16_t*>(alpha)[j]) : static_cast<const float*>(alpha)[j];
}

// alpha[jb..jb+3] (jb a multiple of 4, jb + 4 <= N), branch-free: two 8-byte
// loads (the second repeats the first for f16, where 8 bytes hold all four).
BGB_DEV void alpha4(const void* alpha, int alpha_f16, int64_t jb, float (&al)[4]) {
    const char* ap = static_cast<const char*>(alpha) + (alpha_f16 ? 2 * jb : 4 * jb);
    const uint2 u0 = *reinterpret_cast<const uint2*>(ap);
    const uint2 u1 = *reinterpret_cast<const uint2*>(ap + (alpha_f16 ? 0 : 8));
    al[0] = alpha_f16 ? f16_to_f32(uint16_t(u0.x)) : __uint_as_float(u0.x);
    al[1] = alpha_f16 ? f16_to_f32(uint16_t(u0.x >> 16)) : __uint_as_float(u0.y);
    al[2] = alpha_f16 ? f16_to_f32(uint16_t(u0.y)) : __uint_as_float(u1.x);
    al[3] = alpha_f16 ? f16_to_f32(uint16_t(u0.y >> 16)) : __uint_as_float(u1.y);
}

// Four consecutive outputs jb..jb+3 of one token, o = m * N + jb.
BGB_DEV void store_out16(void* y, int y_dtype, int64_t o, const float (&v)[4], bool full, int64_t jb, int64_t N) {
    if (full && y_dtype == kDtF32) {
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(y) + o) = f32x4_t{v[0], v[1], v[2], v[3]};
    } else if (full) {
        uint16_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = y_dtype == kDtBF16 ? f32_to_bf16_rne(v[i]) : f32_to_f16_rne(v[i]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + o) =
            uint2{uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16)};
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (jb + i >= N) continue;
            if (y_dtype == kDtF32) static_cast<float*>(y)[o + i] = v[i];
            else if (y_dtype == kDtBF16) static_cast<uint16_t*>(y)[o + i] = f32_to_bf16_rne(v[i]);
            else static_cast<uint16_t*>(y)[o + i] = f32_to_f16_rne(v[i]);
        }
    }
}

// The W1A8 epilogue's per-token factors: beta gamma_m / Q_b and the code row
// sum of token m (0 for ternary weights).
BGB_DEV void epi8_token(const GemmArgs& a, bool tern, int64_t m, float& scale, int32_t& rs) {
    scale = (a.beta[0] * a.gamma[m * a.gstride]) / a.qb;
    rs = tern ? 0 : a.rowsum[m];
}

BGB_DEV void store_out8(const GemmArgs& a, bool tern, int64_t o, const i32x4_t& s, float scale, int32_t rs,
                        bool full, int64_t jb) {
    i32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = tern ? s[i] : 2 * s[i] - rs;     // binary: 2 sum b q - sum q
    float* y = static_cast<float*>(a.y);
    if (full) {
        *reinterpret_cast<f32x4_t*>(y + o) =
            f32x4_t{float(v[0]) * scale, float(v[1]) * scale, float(v[2]) * scale, float(v[3]) * scale};
        if (a.acc_opt) *reinterpret_cast<i32x4_t*>(a.acc_opt + o) = v;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (jb + i >= a.N) continue;
            y[o + i] = float(v[i]) * scale;
            if (a.acc_opt) a.acc_opt[o + i] = v[i];
        }
    }
}

// NN token fragments per wave (BM = 16 NN); kW1A8 selects the int8 path;
// kTern (int8 path only) takes ternary weights as two sign planes (+1 plane,
// then -1 plane, each in the binary format) and keeps two accumulator sets.
// kKTail (W1A16, K not a multiple of 128): the stages reaching past K take
// zeros for those activation chunks.
template <bool kW1A8, bool kF16, int NN, int NW, bool kTern = false, bool kKTail = false>
BGB_DEV void gemm_tile(const GemmArgs& a, const int tile, const int z) {
    static_assert(!kTern || kW1A8, "ternary weights take the int8 path");
    static_assert(!kKTail || !kW1A8, "the int8 codes arrive zero-padded");
    constexpr int BM = 16 * NN;
    constexpr int BJ = 64 * NW;                 // 64 columns per wave
    constexpr int kStage = BM * 128;            // bytes of one activation stage
    constexpr int kWTileBytes = BJ * 16;        // one 128-row sign tile of the block's columns
    constexpr int kPlanes = kTern ? 2 : 1;
    constexpr int kXDma = BM / (8 * NW);        // activation DMA operations per thread per stage
    constexpr int kOps = kXDma + kPlanes;       // + the sign tile(s)
    using acc_t = std::conditional_t<kW1A8, i32x4_t, f32x4_t>;
    using opd_t = std::conditional_t<kW1A8, i32x4_t, u32x4_t>;
    constexpr uint32_t kOne = kF16 ? 0x3C003C00u : 0x3F803F80u;

    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t wl0[kWTileBytes * kPlanes];
    __shared__ __attribute__((aligned(1024))) uint8_t wl1[kWTileBytes * kPlanes];
    __shared__ __attribute__((aligned(1024))) uint8_t wl2[kWTileBytes * kPlanes];
    __shared__ __attribute__((aligned(1024))) uint8_t wl3[kWTileBytes * kPlanes];
    uint8_t* const lds[kRing] = {lds0, lds1, lds2, lds3};
    uint8_t* const wls[kRing] = {wl0, wl1, wl2, wl3};

    const int64_t m0 = int64_t(tile / a.ntj) * BM, j0 = int64_t(tile % a.ntj) * BJ;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
    const int s0 = z * a.per;
    const int ns = (s0 + a.per < a.T ? s0 + a.per : a.T) - s0;   // >= 1 by the plan
    const int64_t M = a.M, N = a.N;

    // DMA plan: activation instruction i of wave w moves stage chunks
    // (4i+w)*64 .. +63; lane L takes chunk p -> token row p>>3, LDS slot p&7,
    // source chunk (p&7) ^ swz(row); rows past M read row M-1 (never stored).
    // Thread tid moves column j0 + tid (clamped to N-1) of the sign tile.
    // W1A16 reads x itself: chunks past K (the tail of the last 64-row
    // stage, and stages past K) come from a zero chunk, as their sign bits
    // (0 -> -1) must meet zero activations.
    const uint8_t* src[kXDma];
    auto chunk_of = [&](int i, int& t) {        // source chunk of instruction i for this lane
        const int p = (NW * i + wave) * 64 + lane;
        t = p >> 3;
        return (p & 7) ^ (kW1A8 ? swz8(t) : swz16(t));
    };
#pragma unroll
    for (int i = 0; i < kXDma; ++i) {
        int t;
        const int c = chunk_of(i, t);
        const int64_t m = m0 + t < M ? m0 + t : M - 1;
        src[i] = a.act + m * a.row_bytes + 16 * c;
    }
    const uint8_t* wsrc = reinterpret_cast<const uint8_t*>(a.P + (j0 + tid < N ? j0 + tid : N - 1) * 4);
    auto issue = [&](int rel, int B) {          // stage s0 + rel, clamped: the tail re-reads the last one
        const int s = s0 + (rel < ns ? rel : ns - 1);
#pragma unroll
        for (int i = 0; i < kXDma; ++i) {
            const uint8_t* sp = src[i] + int64_t(s) * 128;
            if constexpr (kKTail) {              // W1A16 with K % 128 != 0: chunks past K read zeros
                int t;
                if (int64_t(s) * 64 + 8 * chunk_of(i, t) >= a.K) sp = reinterpret_cast<const uint8_t*>(g_zero16);
            }
            dma16(sp, lds[B] + (NW * i + wave) * 1024);
        }
        const int64_t tq = kW1A8 ? s : (s >> 1);
        dma16(wsrc + tq * N * 16, wls[B] + wave * 1024);
        if constexpr (kTern) dma16(wsrc + (int64_t(a.T) + tq) * N * 16, wls[B] + kWTileBytes + wave * 1024);
    };

    // B-operand byte offsets in a stage (token row 16n + r) and this lane's
    // sign word. W1A16: half v takes chunk u = 2v + (g & 1) of word g >> 1,
    // i.e. rows 8u..8u+7 of that 32-row word in their natural order.
    int boff0, boff1, wbyte;
    if constexpr (kW1A8) {
        const int rsw = swz8(r);
        boff0 = r * 128 + 16 * ((2 * g) ^ rsw);
        boff1 = r * 128 + 16 * ((2 * g + 1) ^ rsw);
        wbyte = (64 * wave + r) * 16 + 4 * g;                       // + 256 f
    } else {
        const int rsw = swz16(r);
        boff0 = r * 128 + 16 * ((4 * (g >> 1) + (g & 1)) ^ rsw);
        boff1 = r * 128 + 16 * ((4 * (g >> 1) + 2 + (g & 1)) ^ rsw);
        wbyte = (64 * wave + r) * 16 + 4 * (g >> 1);                // + 256 f + 8 (s & 1)
    }
    const uint32_t psel = (g & 1) ? 0x03010301u : 0x02000200u;   // W1A16: bytes (h, h + 2, h, h + 2)

    acc_t acc[4][NN], accn[kTern ? 4 : 1][kTern ? NN : 1];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int n = 0; n < NN; ++n) acc[f][n] = acc_t{0, 0, 0, 0};
    if constexpr (kTern) {
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int n = 0; n < NN; ++n) accn[f][n] = acc_t{0, 0, 0, 0};
    }

    // Operands of the next MFMA group, carried between steps: the sign words
    // (shifted for W1A16) and the v = 0 B fragments of the stage.
    uint32_t X[4], Xn[kTern ? 4 : 1];
    opd_t b0[NN];
    auto load_head = [&](int rel, int B) {
        const int wb = kW1A8 ? wbyte : wbyte + 8 * ((s0 + rel) & 1);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(wls[B] + wb + 256 * f);
            X[f] = (kW1A8 || kKTail) ? w : gather_pairs(w, psel);   // W1A16 with a K tail: at use (registers)
            if constexpr (kTern) Xn[f] = *reinterpret_cast<const uint32_t*>(wls[B] + kWTileBytes + wb + 256 * f);
        }
#pragma unroll
        for (int n = 0; n < NN; ++n) b0[n] = *reinterpret_cast<const opd_t*>(lds[B] + n * 2048 + boff0);
    };
    auto mfma_half = [&](int v, const uint32_t (&Xv)[4], const uint32_t (&Xnv)[kTern ? 4 : 1], const opd_t (&b)[NN]) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            if constexpr (kW1A8) {
                const uint32_t w = Xv[f];
                i32x4_t av;
                av.x = int((w >> (4 * v + 0)) & 0x01010101u);
                av.y = int((w >> (4 * v + 1)) & 0x01010101u);
                av.z = int((w >> (4 * v + 2)) & 0x01010101u);
                av.w = int((w >> (4 * v + 3)) & 0x01010101u);
#pragma unroll
                for (int n = 0; n < NN; ++n)
                    acc[f][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b[n], acc[f][n], 0, 0, 0);
                if constexpr (kTern) {         // the -1 plane into its own accumulators
                    const uint32_t wn = Xnv[f];
                    i32x4_t an;
                    an.x = int((wn >> (4 * v + 0)) & 0x01010101u);
                    an.y = int((wn >> (4 * v + 1)) & 0x01010101u);
                    an.z = int((wn >> (4 * v + 2)) & 0x01010101u);
                    an.w = int((wn >> (4 * v + 3)) & 0x01010101u);
#pragma unroll
                    for (int n = 0; n < NN; ++n)
                        accn[f][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(an, b[n], accn[f][n], 0, 0, 0);
                }
            } else {
                // (~(X << s) & 0x80008000) | one: X holds the lane's rows of
                // the word with rows 8u + 2e and 8u + 2e + 1 (u = 2v + (g & 1))
                // at bits 8v + e and 16 + 8v + e, so dword e gets the sign pair
                // the B operand holds
                u32x4_t av;
                av.x = __builtin_amdgcn_bitop3_b32(Xv[f] << (15 - 8 * v), 0x80008000u, kOne, 0xAE);
                av.y = __builtin_amdgcn_bitop3_b32(Xv[f] << (14 - 8 * v), 0x80008000u, kOne, 0xAE);
                av.z = __builtin_amdgcn_bitop3_b32(Xv[f] << (13 - 8 * v), 0x80008000u, kOne, 0xAE);
                av.w = __builtin_amdgcn_bitop3_b32(Xv[f] << (12 - 8 * v), 0x80008000u, kOne, 0xAE);
#pragma unroll
                for (int n = 0; n < NN; ++n) acc[f][n] = mfma16g<kF16>(av, b[n], acc[f][n]);
            }
        }
    };
    // Step rel: the v = 0 half of the stage runs on operands fetched during
    // the previous step while the v = 1 fragments load; then, once every wave
    // has its reads of this stage back and the next stage has landed, one
    // barrier frees ring slot rel%4 for stage rel+4 and the v = 1 half runs
    // while the next stage's head operands load. Two later stages are in
    // flight behind the next one at that barrier.
    auto step = [&](int rel, auto Bc) {
        constexpr int B = decltype(Bc)::value;
        opd_t b1[NN];
#pragma unroll
        for (int n = 0; n < NN; ++n) b1[n] = *reinterpret_cast<const opd_t*>(lds[B] + n * 2048 + boff1);
        uint32_t Xc[4], Xnc[kTern ? 4 : 1];
#pragma unroll
        for (int f = 0; f < 4; ++f) Xc[f] = (kW1A8 || !kKTail) ? X[f] : gather_pairs(X[f], psel);
        if constexpr (kTern) {
#pragma unroll
            for (int f = 0; f < 4; ++f) Xnc[f] = Xn[f];
        }
        mfma_half(0, Xc, Xnc, b0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt_lgkm0<2 * kOps>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(rel + 4, B);
        load_head(rel + 1, (B + 1) % kRing);
        mfma_half(1, Xc, Xnc, b1);
    };

    issue(0, 0);
    issue(1, 1);
    issue(2, 2);
    issue(3, 3);
    wait_vmcnt<3 * kOps>();
    __builtin_amdgcn_s_barrier();
    load_head(0, 0);
    int rel = 0;
    for (; rel + 4 <= ns; rel += 4) {
        step(rel, std::integral_constant<int, 0>{});
        step(rel + 1, std::integral_constant<int, 1>{});
        step(rel + 2, std::integral_constant<int, 2>{});
        step(rel + 3, std::integral_constant<int, 3>{});
    }
    if (rel < ns) step(rel, std::integral_constant<int, 0>{});
    if (rel + 1 < ns) step(rel + 1, std::integral_constant<int, 1>{});
    if (rel + 2 < ns) step(rel + 2, std::integral_constant<int, 2>{});
    wait_vmcnt<0>();                            // no LDS DMA may outlive the block

    if constexpr (kTern) {                      // sum t q = sum over the +1 plane - sum over the -1 plane
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int n = 0; n < NN; ++n) acc[f][n] -= accn[f][n];
    }
    // Epilogue: lane (g, r) holds columns jb..jb+3 of token 16n + r. Every
    // load it needs (alpha of the lane's 16 columns, or the NN tokens' scale
    // and row sum) is issued before its first store: a wait for a load also
    // waits for every store issued before it, so loads between the stores
    // would make each group of stores wait for the previous one to land.
    float al[4][4], sc[NN];
    int32_t rsum[NN];
    if (!a.part) {
        if constexpr (kW1A8) {
#pragma unroll
            for (int n = 0; n < NN; ++n) {
                const int64_t m = m0 + 16 * n + r;
                epi8_token(a, kTern, m < M ? m : M - 1, sc[n], rsum[n]);   // kTern is a.tern here
            }
        } else {
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int64_t jb = j0 + 64 * wave + 16 * f + 4 * g;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = alpha_at(a.alpha, a.alpha_f16, jb + i < N ? jb + i : N - 1);
                    al[f][i] = jb + i < N ? v : 0.0f;
                }
            }
        }
        wait_vmcnt<0>();                        // (the compiler's own waits would sit between the stores)
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int64_t jb = j0 + 64 * wave + 16 * f + 4 * g;
        const bool full = jb + 4 <= N && (N & 3) == 0;
#pragma unroll
        for (int n = 0; n < NN; ++n) {
            const int64_t m = m0 + 16 * n + r;
            if (m >= M) continue;
            const int64_t o = m * N + jb;
            if (a.part) {                       // raw sums of this split
                const int64_t po = int64_t(z) * M * N + o;
                if (full) {
                    *reinterpret_cast<acc_t*>(static_cast<char*>(a.part) + po * 4) = acc[f][n];
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (jb + i >= N) continue;
                        if constexpr (kW1A8) static_cast<int32_t*>(a.part)[po + i] = acc[f][n][i];
                        else static_cast<float*>(a.part)[po + i] = acc[f][n][i];
                    }
                }
            } else if constexpr (kW1A8) {
                store_out8(a, kTern, o, acc[f][n], sc[n], rsum[n], full, jb);
            } else {
                const float v[4] = {al[f][0] * acc[f][n][0], al[f][1] * acc[f][n][1], al[f][2] * acc[f][n][2],
                                    al[f][3] * acc[f][n][3]};
                store_out16(a.y, a.y_dtype, o, v, full, jb, N);
            }
        }
    }
}

template <bool kW1A8, bool kF16, int NN, int NW, bool kTern = false, bool kKTail = false>
__global__ void __launch_bounds__(NW * 64, 8 / NW) gemm_kernel(const GemmArgs a) {
    const int tile = xcd_tile(blockIdx.x, a.ntiles);
    if (tile >= a.ntiles) return;
    gemm_tile<kW1A8, kF16, NN, NW, kTern, kKTail>(a, tile, blockIdx.y);
}

// Sum of the splits in split order, then the epilogue. One thread per 4
// consecutive columns of one token.
// The K splits' raw sums of one thread's 4 outputs, 8 splits at a time: the
// loads of a batch are in flight together, and the additions run in split
// order (the same sequence as a plain loop). An index past the last split
// re-reads the last one and is not added: branch-free, so the loads stay in
// straight-line code (with a branch per load the compiler waits after each).
template <typename V, typename T>
BGB_DEV void load_splits8(V (&v)[8], const T* p, int z0, int splits, int64_t MN, int64_t o) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int z = z0 + q < splits ? z0 + q : splits - 1;
        v[q] = *reinterpret_cast<const V*>(p + z * MN + o);
    }
}
template <typename V>
BGB_DEV void add_splits8(V& s, const V (&v)[8], int z0, int splits) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
        if (z0 + q < splits) s += v[q];
}

template <bool kW1A8, int kT = 256>
__global__ void __launch_bounds__(kT) splitk_reduce_kernel(const GemmArgs a, int splits) {
    const int64_t M = a.M, N = a.N, nq = (N + 3) / 4;
    const int64_t id = int64_t(blockIdx.x) * kT + threadIdx.x;
    if (id >= M * nq) return;
    const int64_t m = id / nq, jb = 4 * (id % nq), o = m * N + jb;
    const bool full = jb + 4 <= N && (N & 3) == 0;
    const int64_t MN = M * N;
    if constexpr (kW1A8) {
        const int32_t* p = static_cast<const int32_t*>(a.part);
        float scale;
        int32_t rs;
        epi8_token(a, a.tern, m, scale, rs);                // in flight with the first batch
        i32x4_t s = {0, 0, 0, 0};
        if (full) {
            i32x4_t v[8];
            for (int z0 = 0; z0 < splits; z0 += 8) {
                load_splits8(v, p, z0, splits, MN, o);
                add_splits8(s, v, z0, splits);
            }
        } else {
            for (int z = 0; z < splits; ++z)
                for (int i = 0; i < 4; ++i)
                    if (jb + i < N) s[i] += p[z * MN + o + i];
        }
        store_out8(a, a.tern, o, s, scale, rs, full, jb);
    } else {
        const float* p = static_cast<const float*>(a.part);
        float al[4];
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
        if (full) {
            f32x4_t v[8];
            load_splits8(v, p, 0, splits, MN, o);
            alpha4(a.alpha, a.alpha_f16, jb, al);          // in flight with the first batch
            add_splits8(s, v, 0, splits);
            for (int z0 = 8; z0 < splits; z0 += 8) {
                load_splits8(v, p, z0, splits, MN, o);
                add_splits8(s, v, z0, splits);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) al[i] = jb + i < N ? alpha_at(a.alpha, a.alpha_f16, jb + i) : 0.0f;
            for (int z = 0; z < splits; ++z)
                for (int i = 0; i < 4; ++i)
                    if (jb + i < N) s[i] += p[z * MN + o + i];
        }
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = jb + i < N ? al[i] * s[i] : 0.0f;
        store_out16(a.y, a.y_dtype, o, v, full, jb, N);
    }
}

template <bool kW1A8, bool kF16>
static hipError_t launch_gemm(GemmArgs a, const GemmPlan& p, hipStream_t s) {
    const int ntiles = p.ntm * p.ntj;
    a.T = p.T;
    a.per = p.per;
    a.ntj = p.ntj;
    a.ntiles = ntiles;
    const dim3 grid(unsigned(xcd_grid(ntiles)), unsigned(p.splits));
    if constexpr (kW1A8) {
        if (a.tern) {                           // the plan gives 64-token tiles
            gemm_kernel<true, false, 4, 4, true><<<grid, 256, 0, s>>>(a);
            if (p.splits > 1) {
                const int64_t n = a.M * ((a.N + 3) / 4);
                splitk_reduce_kernel<true><<<unsigned((n + 255) / 256), 256, 0, s>>>(a, p.splits);
            }
            return hipGetLastError();
        }
    }
    if constexpr (!kW1A8) {
        if (a.K % 128 != 0) {
            if (p.nn == 8) gemm_kernel<false, kF16, 8, 4, false, true><<<grid, 256, 0, s>>>(a);
            else gemm_kernel<false, kF16, 4, 4, false, true><<<grid, 256, 0, s>>>(a);
            if (p.splits > 1) {
                const int64_t n = a.M * ((a.N + 3) / 4);
                splitk_reduce_kernel<kW1A8><<<unsigned((n + 255) / 256), 256, 0, s>>>(a, p.splits);
            }
            return hipGetLastError();
        }
    }
    if (p.nn == 8) gemm_kernel<kW1A8, kF16, 8, 4><<<grid, 256, 0, s>>>(a);
    else gemm_kernel<kW1A8, kF16, 4, 4><<<grid, 256, 0, s>>>(a);
    if (p.splits > 1) {
        const int64_t n = a.M * ((a.N + 3) / 4);
        splitk_reduce_kernel<kW1A8><<<unsigned((n + 255) / 256), 256, 0, s>>>(a, p.splits);
    }
    return hipGetLastError();
}

// ------------------------------------------------------- grouped, 17..64 ----
// Several independent W1A16 linears of 17 to 64 tokens in one launch (the
// linears of a decoder layer at a decode step). Each item runs the GEMM tile
// above with 64-token tiles (NN = 4); its K range is split into S_i parts so
// that the launch holds enough units of about equal length to fill the chip.
// Items with S_i = 1 write y directly; the others store raw sums, which one
// reduce launch for the whole group adds in part order (so results are the
// same from run to run) before applying the epilogue. Units are numbered
// split-major within an item (the units of one part share activation rows).
struct GemmGroupItem {
    GemmArgs a;
    int first;
};
struct GemmGroup {
    GemmGroupItem it[kGroupMax];
    int count, units;
};

template <bool kF16, bool kKTail>
__global__ void __launch_bounds__(256, 2) gemm_group_kernel(const GemmGroup g) {
    const int u = xcd_tile(blockIdx.x, g.units);
    if (u >= g.units) return;
    GemmGroupItem it = g.it[0];
#pragma unroll
    for (int i = 1; i < kGroupMax; ++i)
        if (i < g.count && u >= g.it[i].first) it = g.it[i];
    const int rel = u - it.first;
    const int z = rel / it.a.ntiles, tile = rel - z * it.a.ntiles;
    gemm_tile<false, kF16, 4, 4, false, kKTail>(it.a, tile, z);
}

// The reduce pass of a group: the items with split K ranges, each over its
// own range of blocks; one thread per 4 consecutive columns of one token.
struct ReduceItem {
    const float* part;
    const void* alpha;
    void* y;
    int64_t M, N;
    int splits, first;      // first block
};
struct ReduceGroup {
    ReduceItem it[kGroupMax];
    int count, alpha_f16, y_dtype;
};

__global__ void __launch_bounds__(256) group_reduce_kernel(const ReduceGroup g) {
    ReduceItem it = g.it[0];
#pragma unroll
    for (int i = 1; i < kGroupMax; ++i)
        if (i < g.count && int(blockIdx.x) >= g.it[i].first) it = g.it[i];
    const int64_t M = it.M, N = it.N, nq = (N + 3) / 4;
    const int64_t id = int64_t(int(blockIdx.x) - it.first) * 256 + threadIdx.x;
    if (id >= M * nq) return;
    const int64_t m = id / nq, jb = 4 * (id % nq), o = m * N + jb;
    const bool full = jb + 4 <= N && (N & 3) == 0;
    const int64_t MN = M * N;
    float al[4];
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
    if (full) {
        f32x4_t v[8];
        load_splits8(v, it.part, 0, it.splits, MN, o);
        alpha4(it.alpha, g.alpha_f16, jb, al);              // in flight with the first batch
        add_splits8(s, v, 0, it.splits);
        for (int z0 = 8; z0 < it.splits; z0 += 8) {
            load_splits8(v, it.part, z0, it.splits, MN, o);
            add_splits8(s, v, z0, it.splits);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = jb + i < N ? alpha_at(it.alpha, g.alpha_f16, jb + i) : 0.0f;
        for (int z = 0; z < it.splits; ++z)
            for (int i = 0; i < 4; ++i)
                if (jb + i < N) s[i] += it.part[z * MN + o + i];
    }
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = jb + i < N ? al[i] * s[i] : 0.0f;
    store_out16(it.y, g.y_dtype, o, v, full, jb, N);
}

namespace {
// Cost model of a grouped launch, in microseconds: per CU, the stages of the
// units it holds (units dealt round-robin to kGroupCUs CUs, kFixedStages of
// fill and epilogue each) at kGroupStageUs per 64-token stage, one unit
// alone on a CU, kGroupSharedUs per stage when two share it; with any split,
// the reduce pass (a launch plus S_i + 1 passes over M x N_i fp32 at
// kGroupReduceBytesPerUs). Fitted to the 1.3B-shaped layer at 64 tokens
// (K split targets of 4 to 32 stages): a stage there costs several times its
// matrix-core work.
constexpr int kGroupCUs = 256;
constexpr double kGroupStageUs = 0.85, kGroupSharedUs = 0.75, kGroupReduceBytesPerUs = 4.0e6;
struct GroupPlan {
    int n, units, order[kGroupMax], splits[kGroupMax], per[kGroupMax], T[kGroupMax], ntj[kGroupMax];
    size_t part_off[kGroupMax], total;
};

GroupPlan group_plan(const W1a16Item* items, int count, int64_t M) {
    GroupPlan g{};
    int tmax = 1;
    for (int i = 0; i < count; ++i) {
        g.T[i] = int(2 * tiles_per_col(items[i].K));           // 64-row stages
        g.ntj[i] = int((items[i].N + 255) / 256);
        tmax = g.T[i] > tmax ? g.T[i] : tmax;
    }
    double best = 1e300;
    int bestP = tmax;
    for (int P = 2; P <= tmax; ++P) {
        int64_t units = 0;
        int maxper = 0;
        double fix = 0.0;
        bool any = false;
        for (int i = 0; i < count; ++i) {
            int S = (g.T[i] + P - 1) / P;
            const int per = (g.T[i] + S - 1) / S;
            S = (g.T[i] + per - 1) / per;
            units += int64_t(g.ntj[i]) * S;
            maxper = per > maxper ? per : maxper;
            if (S > 1) {
                fix += double(S + 1) * double(M) * double(items[i].N) * 4.0;
                any = true;
            }
        }
        const int64_t per_cu = (units + kGroupCUs - 1) / kGroupCUs;      // units on the busiest CU
        double t = per_cu <= 1 ? (maxper + kFixedStages) * kGroupStageUs
                               : double(per_cu) * (maxper + kFixedStages) * kGroupSharedUs;
        if (any) t += kLaunchUs + fix / kGroupReduceBytesPerUs;
        if (t < best - 1e-9) {
            best = t;
            bestP = P;
        }
    }
    for (int i = 0; i < count; ++i) {
        const int S = (g.T[i] + bestP - 1) / bestP;
        g.per[i] = (g.T[i] + S - 1) / S;
        g.splits[i] = (g.T[i] + g.per[i] - 1) / g.per[i];
        g.order[i] = i;
    }
    // the longest units first
    for (int a = 1; a < count; ++a)
        for (int b = a; b > 0 && g.per[g.order[b]] > g.per[g.order[b - 1]]; --b) {
            const int t = g.order[b];
            g.order[b] = g.order[b - 1];
            g.order[b - 1] = t;
        }
    size_t part = 0;
    int64_t units = 0;
    for (int i = 0; i < count; ++i) {
        g.part_off[i] = part;
        if (g.splits[i] > 1) part += align256(size_t(g.splits[i]) * size_t(M) * size_t(items[i].N) * 4);
        units += int64_t(g.ntj[i]) * g.splits[i];
    }
    g.n = count;
    g.total = part;
    g.units = int(units);
    return g;
}
}  // namespace

bool w1a16_gemm_group_supported(const W1a16Item* items, int count, int64_t M) {
    if (M < 17 || M > 64 || count < 1 || count > kGroupMax) return false;
    int64_t units = 0;
    for (int i = 0; i < count; ++i) {
        if (items[i].K <= 0 || items[i].N <= 0) return false;
        units += (items[i].N + 255) / 256 * 2 * tiles_per_col(items[i].K);
    }
    return units < (int64_t(1) << 30);
}

size_t w1a16_gemm_group_ws_bytes(const W1a16Item* items, int count, int64_t M) {
    if (!w1a16_gemm_group_supported(items, count, M)) return 0;
    return group_plan(items, count, M).total;
}

hipError_t launch_w1a16_gemm_group(const W1a16Item* items, int count, int64_t M, int x_f16, int alpha_f16,
                                   int y_dtype, void* ws, hipStream_t s) {
    if (!w1a16_gemm_group_supported(items, count, M)) return hipErrorInvalidValue;
    const GroupPlan p = group_plan(items, count, M);
    if (p.total && !ws) return hipErrorInvalidValue;
    GemmGroup h{};
    ReduceGroup rg{};
    int first = 0, rfirst = 0, nr = 0;
    bool tail = false;
    for (int k = 0; k < count; ++k) {
        const int i = p.order[k];
        const W1a16Item& in = items[i];
        GemmArgs& a = h.it[k].a;
        a.act = static_cast<const uint8_t*>(in.x);
        a.row_bytes = in.K * 2;
        a.K = in.K;
        a.P = in.P;
        a.M = M;
        a.N = in.N;
        a.T = p.T[i];
        a.per = p.per[i];
        a.ntj = p.ntj[i];
        a.ntiles = p.ntj[i];                              // one 64-token tile row
        a.alpha = in.alpha;
        a.alpha_f16 = alpha_f16;
        a.y = in.y;
        a.y_dtype = y_dtype;
        a.part = p.splits[i] > 1 ? static_cast<char*>(ws) + p.part_off[i] : nullptr;
        h.it[k].first = first;
        first += p.ntj[i] * p.splits[i];
        tail |= (in.K % 128) != 0;
        if (p.splits[i] > 1) {
            ReduceItem& r = rg.it[nr++];
            r.part = static_cast<const float*>(a.part);
            r.alpha = in.alpha;
            r.y = in.y;
            r.M = M;
            r.N = in.N;
            r.splits = p.splits[i];
            r.first = rfirst;
            rfirst += int((M * ((in.N + 3) / 4) + 255) / 256);
        }
    }
    h.count = count;
    h.units = first;
    const unsigned grid = unsigned(xcd_grid(first));
    if (x_f16) {
        if (tail) gemm_group_kernel<true, true><<<grid, 256, 0, s>>>(h);
        else gemm_group_kernel<true, false><<<grid, 256, 0, s>>>(h);
    } else {
        if (tail) gemm_group_kernel<false, true><<<grid, 256, 0, s>>>(h);
        else gemm_group_kernel<false, false><<<grid, 256, 0, s>>>(h);
    }
    if (nr) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        rg.count = nr;
        rg.alpha_f16 = alpha_f16;
        rg.y_dtype = y_dtype;
        group_reduce_kernel<<<unsigned(rfirst), 256, 0, s>>>(rg);
    }
    return hipGetLastError();
}

hipError_t launch_w1a16_splitk_reduce(const float* part, int splits, int64_t M, int64_t N, const void* alpha,
                                      int alpha_f16, void* y, int y_dtype, hipStream_t s) {
    GemmArgs a{};
    a.M = M;
    a.N = N;
    a.alpha = alpha;
    a.alpha_f16 = alpha_f16;
    a.y = y;
    a.y_dtype = y_dtype;
    a.part = const_cast<float*>(part);
    const int64_t n = M * ((N + 3) / 4);
    // one wave per block: at decode sizes (M x N / 4 threads, 16K at 16 tokens
    // x 4096 columns) the pass is a single round of loads, spread over 4x the CUs
    splitk_reduce_kernel<false, 64><<<unsigned((n + 63) / 64), 64, 0, s>>>(a, splits);
    return hipGetLastError();
}

hipError_t launch_w1a16_gemm(const uint16_t* x, int x_f16, int64_t M, int64_t K, int64_t N, const uint32_t* P,
                             const void* alpha, int alpha_f16, void* y, int y_dtype, void* part, hipStream_t s) {
    const GemmPlan p = gemm_plan(M, K, N, false, false);
    GemmArgs a{};
    a.act = reinterpret_cast<const uint8_t*>(x);
    a.row_bytes = K * 2;
    a.K = K;
    a.P = P;
    a.M = M;
    a.N = N;
    a.alpha = alpha;
    a.alpha_f16 = alpha_f16;
    a.y = y;
    a.y_dtype = y_dtype;
    a.part = p.splits > 1 ? part : nullptr;
    return x_f16 ? launch_gemm<false, true>(a, p, s) : launch_gemm<false, false>(a, p, s);
}

hipError_t launch_w1a8_gemm(const int8_t* q, const int32_t* rowsum, const float* gamma, int gstride,
                            const float* beta, float qb,
                            int64_t M, int64_t K, int64_t N, const uint32_t* P, float* y, int32_t* acc_opt,
                            void* part, int tern, hipStream_t s) {
    const GemmPlan p = gemm_plan(M, K, N, true, tern != 0);
    GemmArgs a{};
    a.act = reinterpret_cast<const uint8_t*>(q);
    a.row_bytes = padded_k(K);
    a.K = padded_k(K);
    a.P = P;
    a.M = M;
    a.N = N;
    a.rowsum = rowsum;
    a.gamma = gamma;
    a.gstride = gstride;
    a.beta = beta;
    a.qb = qb;
    a.y = y;
    a.acc_opt = acc_opt;
    a.tern = tern;
    a.part = p.splits > 1 ? part : nullptr;
    return launch_gemm<true, false>(a, p, s);
}

}  // namespace bgb
