// Decode kernels (M <= 32): stream the packed signs once from HBM and run the
// contraction on the matrix cores, tokens padded to 16-token fragments.
//
// FBI-linear W1A16 (FBI-LLM news rewrite, FBI-linear paragraph):
//   y[m][j] = alpha_j * sum_k s_kj x[m][k]
// BitLinear W1A8 ("BitNet b1.58: 1bit LLM时代", section 一, eq. (4)-(8)):
//   acc[m][j] = sum_k s_kj q[m][k];  y = acc * beta * gamma / Q_b
//
// Work split: a block of 4 waves owns 16 output columns. The column's tiles
// are taken 4 at a time ("steps" of 512 rows): in a step, lane group g (lanes
// 16g..16g+15) loads the 16-byte tile (4 words, 128 rows) of column
// j0 + (lane % 16) from tile 4*step + g, so one load instruction moves 1 KB.
// Wave w takes steps w, w+4, w+8, ... and issues the loads of up to 8 of its
// steps before it decodes any of them, so a whole layer's signs are in flight
// at once. The MFMA A operand is decoded from these words in registers (rows
// of A = output columns), the B operand holds 16 tokens' activations; the 4
// waves' partial sums are added in a fixed order through LDS.
//
// Sign decoding keeps the per-weight work to one bitwise op per 2 or 4 weights:
// * W1A8: with b = 1 for +1, sum_k s q = 2 sum_k b q - sum_k q. The int8 MFMA
//   for shift s takes bytes (word & (0x01010101 << s)) -- 2^s b, or -128 b for
//   s = 7 -- from the 4 words of the tile, so it accumulates 2^s sum b q
//   exactly; the 8 accumulators are shifted back and added.
// * W1A16: a 16-bit float whose exponent field is set and one low field bit b
//   free encodes a + c b. MFMA u (0..15) takes bit u and bit u + 16 of each
//   word, moved by a per-u constant shift into field bit p = P0 + u % 4 (one
//   shift per word serves four MFMAs): p = P0..P0+2 are mantissa bits over a
//   base of 1.0 (a = 1; c = 1/8, 1/4, 1/2), p = P0+3 is the exponent's lowest
//   bit over a base of 0.5 (a = 1/2, c = 1/2). MFMAs of one type T = u % 4
//   share an accumulator acc_T = a_T X_T + c_T sum_{k in T} b x, with X_T the
//   sum of x over the rows of type T (k % 4 == T), so
//   sum_k b x = sum_T (acc_T - a_T X_T) / c_T, all scalings powers of two.
//
// Single-token calls (M == 1, the common decode case) fuse the activation
// side into the same launch: every block first issues its weight loads, then
// builds the activation operand in LDS (BitLinear: LayerNorm, absmax and the
// int8 codes; FBI-linear: the permuted bf16/f16 row and the four X_T) while
// the signs are in flight. Each block repeats that small prologue; its
// results are identical in every block.
#include "bgb_device.hpp"
#include "bgb_internal.hpp"

#include <type_traits>

namespace bgb {


// ------------------------------------------------------------ shared bits ----

// Position of activation row k in the W1A8 decode layout (int8, per 128-row
// tile: [s = k%8][d = t%4][e = (k%32)/8] with t = k/32).
BGB_DEV int q_pos(int64_t k) {
    const int64_t t = k >> 5;
    const int b = int(k & 31);
    return int((t >> 2) * 128) + (b & 7) * 16 + int(t & 3) * 4 + (b >> 3);
}
// Position of activation row k in the W1A16 decode layout (16-bit elements,
// per 128-row tile: [u = k%16][d = t%4][h = (k%32)/16]).
BGB_DEV int x_pos(int64_t k) {
    const int64_t t = k >> 5;
    const int b = int(k & 31);
    return int((t >> 2) * 128) + (b & 15) * 8 + int(t & 3) * 2 + (b >> 4);
}

BGB_DEV u32x4_t load_tile(const uint32_t* P, int64_t tq, int64_t N, int64_t j) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(P + (tq * N + j) * 4));
}

// Preload the tiles of S steps of this wave (steps base, base + stride, ...;
// zeros past the end). Every load is issued unconditionally -- an invalid
// step reads tile 0 of column 0 and is zeroed by a select -- so the loads sit
// in straight-line code and the compiler can wait for exactly the ones it
// needs (a skipped load would force it to wait for all of them).
template <int S>
BGB_DEV void preload(u32x4_t* w, const uint32_t* P, int64_t base, int64_t stride, int64_t steps, int64_t TQ,
                     int64_t N, int64_t j, int g) {
#pragma unroll
    for (int i = 0; i < S; ++i) {
        const int64_t st = base + stride * i;
        const int64_t tq = st * 4 + g;
        const bool ok = st < steps && tq < TQ && j < N;
        const uint32_t keep = 0u - uint32_t(ok);
        const u32x4_t t = load_tile(P, ok ? tq : 0, N, ok ? j : 0);
        w[i] = t & keep;
    }
}

// Tiles as preload() reads them, but never masked: a tile past the column's
// last one, or of a column past N, is read from tile 0 of column 0 instead
// (always in bounds). The caller pairs such steps with zero codes and never
// stores such columns. One 64-bit lane address, wave-uniform strides (base and
// stride must be wave-uniform), one select per tile.
template <int S>
BGB_DEV void preload_nomask(u32x4_t* w, const uint32_t* P, int base, int stride, int steps, int TQ, int64_t N,
                            int64_t j, int g) {
    const char* pb = reinterpret_cast<const char*>(P);
    const char* lane0 = pb + ((int64_t(base) * 4 + g) * N + j) * 16;
    const int64_t sb = int64_t(stride) * 64 * N;
    const bool jok = j < N;
    const int room = TQ - g;                           // tile 4 st + g exists iff 4 st < room
#pragma unroll
    for (int i = 0; i < S; ++i) {
        const int st = base + stride * i;
        const bool ok = jok && st < steps && 4 * st < room;
        w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(ok ? lane0 + sb * i : pb));
    }
}

// 16 bytes at p if ok, else zeros -- branch-free (p must be readable either way).
template <typename V>
BGB_DEV V ld16_or0(const V* p, bool ok) {
    const V t = *p;
    return t & V(0 - int(ok));
}

BGB_DEV void store_y(void* y, int y_dtype, int64_t i, float v) {
    if (y_dtype == kDtF32) static_cast<float*>(y)[i] = v;
    else if (y_dtype == kDtBF16) static_cast<uint16_t*>(y)[i] = f32_to_bf16_rne(v);
    else static_cast<uint16_t*>(y)[i] = f32_to_f16_rne(v);
}

BGB_DEV float load_alpha(const void* alpha, int alpha_f16, int64_t j) {
    return alpha_f16 ? f16_to_f32(static_cast<const uint16_t*>(alpha)[j]) : static_cast<const float*>(alpha)[j];
}
BGB_DEV float load_alpha_ahead(const void* alpha, int alpha_f16, int64_t j) {
    const int64_t off = alpha_f16 ? (2 * j) & ~int64_t(3) : 4 * j;
    const uint32_t u = *reinterpret_cast<const uint32_t*>(static_cast<const char*>(alpha) + off);
    return alpha_f16 ? f16_to_f32(uint16_t(u >> (16 * (j & 1)))) : __uint_as_float(u);
}

// ------------------------------------------------------------------ W1A8 -----

template <int S>
BGB_DEV i32x4_t w1a8_mfma(const u32x4_t& w, const i32x4_t& b, const i32x4_t& c) {
    constexpr uint32_t mask = 0x01010101u << S;
    const i32x4_t a = {int(w.x & mask), int(w.y & mask), int(w.z & mask), int(w.w & mask)};
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

BGB_DEV void w1a8_step(const u32x4_t& w, const i32x4_t* b, i32x4_t* acc) {
    acc[0] = w1a8_mfma<0>(w, b[0], acc[0]);
    acc[1] = w1a8_mfma<1>(w, b[1], acc[1]);
    acc[2] = w1a8_mfma<2>(w, b[2], acc[2]);
    acc[3] = w1a8_mfma<3>(w, b[3], acc[3]);
    acc[4] = w1a8_mfma<4>(w, b[4], acc[4]);
    acc[5] = w1a8_mfma<5>(w, b[5], acc[5]);
    acc[6] = w1a8_mfma<6>(w, b[6], acc[6]);
    acc[7] = w1a8_mfma<7>(w, b[7], acc[7]);
}

// Single-token W1A8 product on the fp4 (e2m1) matrix cores, 16 x 16 x 128.
// A holds signs as fp4 nibbles. MFMA type p (0..3) takes bit 4n + p of each of
// the tile's four words into nibble n of the matching dword (rows 32d + 4n + p
// of the tile, d = the word). Type 3 leaves the bit where it is, the sign
// field of 1.0: a set bit gives +1, a clear one -1. Types 0..2 keep the bit as
// the only set field bit of the nibble, 0.5, 1.0 or 2.0 times b (b = 1 for
// +1), so sum_k s q = 2 sum_k b q - sum_k q over those rows. B holds a code q
// as four base-4 digits of |q|, one per token column 0..3 (nibble codes 0..3
// are the fp4 values 0, 0.5, 1, 1.5, so column c carries digit / 2) with q's
// sign in bit 3. Every product and partial sum is a multiple of 1/4 below
// 2^22, so the fp32 accumulators hold them exactly.
typedef int i32x8_t __attribute__((ext_vector_type(8)));
template <int P>
BGB_DEV i32x4_t f4_signs(const u32x4_t& w) {
    if constexpr (P == 3) {   // (~w & 0x88888888) | 0x22222222: +-1.0 per nibble (truth table 0xAE)
        return i32x4_t{int(__builtin_amdgcn_bitop3_b32(w.x, 0x88888888u, 0x22222222u, 0xAE)),
                       int(__builtin_amdgcn_bitop3_b32(w.y, 0x88888888u, 0x22222222u, 0xAE)),
                       int(__builtin_amdgcn_bitop3_b32(w.z, 0x88888888u, 0x22222222u, 0xAE)),
                       int(__builtin_amdgcn_bitop3_b32(w.w, 0x88888888u, 0x22222222u, 0xAE))};
    } else {
        constexpr uint32_t m = 0x11111111u << P;
        return i32x4_t{int(w.x & m), int(w.y & m), int(w.z & m), int(w.w & m)};
    }
}
BGB_DEV f32x4_t mfma_f4(const i32x4_t& a, const i32x4_t& b, const f32x4_t& c) {
    const i32x8_t a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};   // fp4 operands use the first four dwords
    const i32x8_t b8 = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 4, 0, 127, 0, 127);   // scales 2^0
}
// One 512-row step: the four types against the lane's digit operands b[p].
BGB_DEV void w1a8_f4_step(const u32x4_t& w, const i32x4_t* b, f32x4_t* acc) {
    acc[0] = mfma_f4(f4_signs<0>(w), b[0], acc[0]);
    acc[1] = mfma_f4(f4_signs<1>(w), b[1], acc[1]);
    acc[2] = mfma_f4(f4_signs<2>(w), b[2], acc[2]);
    acc[3] = mfma_f4(f4_signs<3>(w), b[3], acc[3]);
}
// Per lane (digit column r of output rows 4g..4g+3): 2 sum b q over types 0..2
// plus sum s q over type 3, for digit r, scaled by its weight 4^r; then summed
// over the quad of digit columns 0..3. Exact (integers below 2^24).
BGB_DEV i32x4_t w1a8_f4_combine(const f32x4_t* acc, int r) {
    const f32x4_t z = ((8.0f * acc[0] + 4.0f * acc[1]) + 2.0f * acc[2]) + 2.0f * acc[3];
    const float wt = r < 4 ? float(1 << (2 * r)) : 0.0f;
    i32x4_t t;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v = z[i] * wt;
        v += dpp_f32<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
        v += dpp_f32<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
        t[i] = int(v);
    }
    return t;
}

// sum_k b q from the 8 shift accumulators (each division by 2^s is exact).
BGB_DEV i32x4_t w1a8_combine(const i32x4_t* acc) {
    i32x4_t t;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int v = 0;
#pragma unroll
        for (int s = 0; s < 7; ++s) v += acc[s][i] >> s;
        t[i] = v - (acc[7][i] >> 7);
    }
    return t;
}

// General decode: codes from the prologue in the decode layout, M <= 16 * TF.
// A block of kGenWaves waves owns 16 columns; each wave takes up to
// kGenSteps steps per pass, loads all their tiles first, decodes each step's
// A operand once and reuses it for the TF token fragments.
constexpr int kGenWaves = 8;
// steps per wave and pass: the fewest that cover the column (at most 4)
inline int gen_steps(int64_t TQ) {
    const int64_t steps = (TQ + 3) / 4;
    return steps <= kGenWaves ? 1 : (steps <= 2 * kGenWaves ? 2 : 4);
}

// kTern: ternary weights as two planes (+1 at P, -1 at Pn); the product is
// then sum_plus - sum_minus and needs no code row sums.
template <int TF, int GS, bool kTern>
__global__ void __launch_bounds__(kGenWaves * 64)
gemv_w1a8_kernel(const int8_t* __restrict__ q, const int32_t* __restrict__ rowsum, const float* __restrict__ gamma,
                 int gstride, const float* __restrict__ beta, float qb, int M, int64_t N, int64_t TQ,
                 const uint32_t* __restrict__ P, float* __restrict__ y, int32_t* __restrict__ acc_opt) {
    __shared__ i32x4_t red[kGenWaves][TF][64];
    const uint32_t* Pn = P + TQ * N * 4;                // -1 plane (ternary)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int64_t j0 = int64_t(blockIdx.x) * 16, j = j0 + r;
    const int64_t Kp = TQ * 128, steps = (TQ + 3) / 4;
    i32x4_t acc[TF][8], accn[kTern ? TF : 1][8];
#pragma unroll
    for (int tf = 0; tf < TF; ++tf)
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) acc[tf][s8] = i32x4_t{0, 0, 0, 0};
    if constexpr (kTern) {
#pragma unroll
        for (int tf = 0; tf < TF; ++tf)
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8) accn[tf][s8] = i32x4_t{0, 0, 0, 0};
    }
    for (int64_t base = wave; base < steps; base += kGenWaves * GS) {
        u32x4_t w[GS], wn[kTern ? GS : 1];
        preload<GS>(w, P, base, kGenWaves, steps, TQ, N, j, g);
        if constexpr (kTern) preload<GS>(wn, Pn, base, kGenWaves, steps, TQ, N, j, g);
#pragma unroll
        for (int i = 0; i < GS; ++i) {
            const int64_t st = base + kGenWaves * i;
            const int64_t tq = st * 4 + g;
            const bool tv = st < steps && tq < TQ;
#pragma unroll
            for (int tf = 0; tf < TF; ++tf) {
                const int m = 16 * tf + r;
                const bool bv = tv && m < M;
                const i32x4_t* src = reinterpret_cast<const i32x4_t*>(q + int64_t(bv ? m : 0) * Kp + (bv ? tq : 0) * 128);
                i32x4_t b[8];
#pragma unroll
                for (int s8 = 0; s8 < 8; ++s8) b[s8] = ld16_or0(src + s8, bv);
                __builtin_amdgcn_sched_barrier(0);   // all 8 operand loads in flight before the MFMAs
                w1a8_step(w[i], b, acc[tf]);
                if constexpr (kTern) w1a8_step(wn[i], b, accn[tf]);
            }
        }
    }
#pragma unroll
    for (int tf = 0; tf < TF; ++tf) {
        red[wave][tf][lane] = w1a8_combine(acc[tf]);
        if constexpr (kTern) red[wave][tf][lane] -= w1a8_combine(accn[tf]);
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int tf = 0; tf < TF; ++tf) {
        const int mm = 16 * tf + r;
        if (mm >= M) continue;
        const float scale = (beta[0] * gamma[int64_t(mm) * gstride]) / qb;   // the tensor's or the token's gamma
        i32x4_t sum = red[0][tf][lane];
#pragma unroll
        for (int wv = 1; wv < kGenWaves; ++wv) sum += red[wv][tf][lane];
        const int32_t rs = kTern ? 0 : rowsum[mm];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t col = j0 + 4 * g + i;
            if (col >= N) continue;
            const int32_t a = kTern ? sum[i] : 2 * sum[i] - rs;   // binary: sum s q = 2 sum b q - sum q
            y[int64_t(mm) * N + col] = float(a) * scale;
            if (acc_opt) acc_opt[int64_t(mm) * N + col] = a;
        }
    }
}

// Single token, prologue fused: x [K] (float or bf16 bits), K <= 1024 * NV.
template <typename XT> BGB_DEV float load1(const XT* x, int64_t k);
template <> BGB_DEV float load1<float>(const float* x, int64_t k) { return x[k]; }
template <> BGB_DEV float load1<uint16_t>(const uint16_t* x, int64_t k) { return __uint_as_float(uint32_t(x[k]) << 16); }

constexpr int kFusedMaxKp = 16384;

// Single-token kernels: a block of NW waves takes column groups of F
// 16-column fragments; wave w works on fragment w % F over the K part
// kq = w / F of KQ = NW / F (steps kq, kq + KQ, ...). Each block runs the
// activation prologue once and then its IT groups, blockIdx.x + i gridDim.x.
constexpr int kD1Waves = 8;         // W1A16 single-token blocks
constexpr int kD1MaxGrid = 256;     // one block per CU
constexpr int kD1MaxTiles = 8;      // preloaded 16-byte sign tiles per thread (IT x S)

// Code of one activation, h already LayerNormed: trunc (or, rne, the nearest
// integer, clamped) of clip(fl32(h Q_b / gamma), +-lim), lim in (Q_b - 1, Q_b).
template <bool kRne>
BGB_DEV int exact_code(float h, float qb, float gamma, float lim) {
    const float v = fminf(fmaxf((h * qb) / gamma, -lim), lim);
    if constexpr (kRne) return round_code(v, true, int(qb) - 1);
    else return int(v);
}

// W1A8 steps per wave: NV dwords of codes per thread cover NV NW / 2 steps of
// 512 rows, shared by KQ = NW / F waves.
constexpr int w1a8_d1_steps(int nv, int f) { return (nv * f + 1) / 2; }

// kTern: ternary weights (BitNet b1.58) as two planes, +1 at P and -1 at
// P + TQ N 4 words; the product is sum_plus - sum_minus (no code row sum).
template <int NV, int NW, int F, int IT, typename XT, bool kRne, bool kTern>
__global__ void __launch_bounds__(NW * 64)
bitlinear_decode1_kernel(const XT* __restrict__ x, int64_t K, double rk, int64_t N, int64_t TQ, double eps, float qb,
                         float lim,
                         const uint32_t* __restrict__ P, const float* __restrict__ beta, float* __restrict__ y,
                         int32_t* __restrict__ acc_opt, int8_t* __restrict__ xq_opt,
                         float* __restrict__ gamma_opt) {
    constexpr int NT = NW * 64;
    constexpr int KQ = NW / F;
    constexpr int S = w1a8_d1_steps(NV, F);
    static_assert(NW % F == 0 && IT * S * (kTern ? 2 : 1) <= kD1MaxTiles, "single-token W1A8 shape");
    // binary weights with two or more code dwords per thread: the fp4 product
    // (a thread then owns octets of rows instead of pairs, see below)
    constexpr bool kF4 = !kTern && NV % 2 == 0;
    // codes (int8: 128 B per 128-row tile; fp4 digits: 256 B), then one zero tile
    __shared__ __attribute__((aligned(16))) int8_t qs[(kF4 ? 2 : 1) * (kFusedMaxKp + 128)];
    __shared__ i32x4_t red[KQ > 1 ? 2 : 1][KQ > 1 ? NW : 1][64];
    __shared__ double dsum[NW], dsq[NW], dsq2[NW];
    __shared__ uint32_t dmx[NW], dmn[NW];
    __shared__ int iscr[NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15, f = wave % F, kq = wave / F;
    const int64_t ngroups = (N + 16 * F - 1) / (16 * F);
    const int Kp = int(TQ * 128);
    const int64_t steps = (TQ + 3) / 4;
    const int pairs = int(K / 4);                      // (t, s): rows 32t + s + 8c, c = 0..3
    // fp4 form: octet o = (t, p) = (o / 4, o % 4) holds rows 32t + p + 4n,
    // n = 0..7; thread tid owns octets h NT + tid, h < NV / 2, and v[2h + e][c]
    // holds n = 2c + e
    const int octets = int(K / 8);
    auto valid = [&](int i) { return kF4 ? (i >> 1) * NT + tid < octets : i * NT + tid < pairs; };

    // 1. the token (an L2 hit after the first block): thread tid owns the
    //    pairs p = i * NT + tid, i.e. the rows of one dword of the decode
    //    layout each. A pair past K loads rows 0, 8, 16, 24 instead (K is a
    //    multiple of 32): real values of the row, so they may enter the
    //    extremes unmasked; the sums take them as zeros, and their codes are
    //    never stored. The loads complete before any sign tile is requested;
    //    the tiles are then in flight during the whole prologue.
    float v[NV][4];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        int64_t k0;
        if constexpr (kF4) {
            const int o = (i >> 1) * NT + tid;       // an octet past K loads rows 4e + 8c of word 0
            k0 = int64_t(o < octets ? 32 * (o >> 2) + (o & 3) : 0) + 4 * (i & 1);
        } else {
            const int p = i * NT + tid;
            k0 = p < pairs ? int64_t(32 * (p >> 3) + (p & 7)) : 0;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) v[i][c] = load1(x, k0 + 8 * c);
    }
    // beta is requested now, beside the token; it and the output pointers
    // (argument slots on a later cache line than the first ones) are pinned
    // in registers after the first barrier below. Left alone, the compiler
    // loads them after the last product, two scalar round trips in front of
    // the stores.
    const float beta0 = beta[0];
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));     // vmcnt(0): the token is in
    // the sign tiles of all of this block's column groups (unmasked: steps
    // past the column's tiles meet the zero code tile, columns past N are
    // never stored)
    u32x4_t w[IT][S], wn[kTern ? IT : 1][S];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int64_t jj = (int64_t(blockIdx.x) + int64_t(it) * gridDim.x) * 16 * F + 16 * f + r;
        preload_nomask<S>(w[it], P, kq, KQ, int(steps), int(TQ), N, jj, g);
        if constexpr (kTern) preload_nomask<S>(wn[it], P + TQ * N * 4, kq, KQ, int(steps), int(TQ), N, jj, g);
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. LayerNorm statistics; every block computes the same values. One pass
    //    gives sum x and sum x^2 in fp64 (x^2 is exact there, so the fused
    //    multiply-add rounds once, as a product and a sum would) and the row's
    //    extreme x. Var = E x^2 - (E x)^2 differs from the exact variance by
    //    at most dv = (3 K + 8) 2^-53 E x^2 (each sum's error is below
    //    K 2^-53 times its sum of magnitudes, |E x| E|x| <= E x^2, plus the
    //    roundings of the quotients, the square and the difference), so
    //    rs32 = fl32(1/sqrt(Var + eps)) is the two-pass value unless
    //    1/sqrt(Var + eps) lies within its propagated error of a point where
    //    the fp32 rounding changes; then (rare, and the same decision in every
    //    thread) the second fp64 pass over (x - mu)^2 decides, as before.
    //    gamma = max |h| with h = fl32(fl32(x - mu32) rs32): rounding is
    //    monotone and sign-symmetric, so gamma = fl32(a rs32) with
    //    a = max |fl32(x - mu32)|, which sits at the largest or smallest x.
    //    The extremes travel as order-preserving integer keys (the minimum as
    //    the maximum of complemented keys), one max per DPP step.
    double s1 = 0.0, s2 = 0.0;
    float xmx = v[0][0], xmn = v[0][0];
    auto pass1 = [&](auto masked) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const bool ok = !decltype(masked)::value || valid(i);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const double d = ok ? double(v[i][c]) : 0.0;
                s1 += d;
                s2 = __builtin_fma(d, d, s2);
                xmx = fmaxf(xmx, v[i][c]);
                xmn = fminf(xmn, v[i][c]);
            }
        }
    };
    if (pairs >= NV * NT) pass1(std::false_type{});      // every pair inside K (uniform)
    else pass1(std::true_type{});
    s1 = wave_sum63(s1);
    s2 = wave_sum63(s2);
    const uint32_t kmx = wave_umax63(f32_sort_key(xmx));
    const uint32_t kmn = wave_umax63(~f32_sort_key(xmn));
    if (lane == 63) {
        dsum[wave] = s1;
        dsq[wave] = s2;
        dmx[wave] = kmx;
        dmn[wave] = kmn;
    }
    __syncthreads();
    asm volatile("" ::"s"(beta0), "s"(y), "s"(acc_opt));
    const double sx = tree_sum<NW>(dsum), sxx = tree_sum<NW>(dsq);
    uint32_t khx = dmx[0], klx = dmn[0];
#pragma unroll
    for (int wv = 1; wv < NW; ++wv) {
        khx = max(khx, dmx[wv]);
        klx = max(klx, dmn[wv]);
    }
    const float hx = f32_from_sort_key(khx), lx = f32_from_sort_key(~klx);
    // the quotients by K correctly rounded without a division: q = sx rk
    // with rk = fl(1/K) is within an ulp, and one correction with the exact
    // remainder fma(-q, K, sx) gives the rounded quotient (Markstein)
    const double kd = double(K);
    const double q1 = sx * rk, q2 = sxx * rk;
    const double mu = __builtin_fma(__builtin_fma(-q1, kd, sx), rk, q1);
    const float mu32 = float(mu);
    const double ex2 = __builtin_fma(__builtin_fma(-q2, kd, sxx), rk, q2);
    const double ve = fmax(ex2 - mu * mu, 0.0) + eps;
    // 1/sqrt(ve): the hardware estimate r0 and one third-order step,
    // r = r0 (1 + e/2 + 3 e^2/8) with e = 1 - ve r0^2. Whatever r0's
    // accuracy, the residual e1 = 1 - ve r^2 bounds r's relative error by
    // 0.5000001 |e1| + 2^-52 while |e1| <= 2^-30; a larger residual (or a
    // non-finite ve) counts as near a boundary and takes the second pass.
    const double r0 = __builtin_amdgcn_rsq(ve);
    const double e0 = __builtin_fma(-(ve * r0), r0, 1.0);
    const double rd = __builtin_fma(r0 * e0, __builtin_fma(e0, 0.375, 0.5), r0);
    const double e1 = fabs(__builtin_fma(-(ve * rd), rd, 1.0));
    float rs32;
    {
        // rd's relative error bound: the one-pass variance's (ex2 rd^2
        // stands for ex2 / ve; the half-unit in the constant covers that),
        // the refinement's, 2^-50 for the eps sum, and 2^-51 for forming the
        // interval's ends. If both ends round to the same fp32 value, so
        // does every point between them (rounding is monotone).
        const double rerr = (1.5 * kd + 4.5) * 0x1p-53 * (ex2 * (rd * rd)) + 0.5000001 * e1 + (0x1p-50 + 0x1p-51);
        const double dr = rd * rerr;
        const float lo = float(rd - dr), hi = float(rd + dr);
        rs32 = hi;
        if (!(lo == hi && e1 <= 0x1p-30)) {
            double q2s = 0.0;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                if (!valid(i)) continue;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const double d = double(v[i][c]) - mu;
                    q2s += d * d;
                }
            }
            q2s = wave_sum63(q2s);
            if (lane == 63) dsq2[wave] = q2s;
            __syncthreads();
            double v2 = dsq2[0];
#pragma unroll
            for (int wv = 1; wv < NW; ++wv) v2 += dsq2[wv];
            rs32 = float(1.0 / sqrt(v2 / kd + eps));
        }
    }
    const float amx = fmaxf(fabsf(hx - mu32), fabsf(lx - mu32));
    const float gamma = amx * rs32;

    // 3. codes into LDS in the decode layout, one dword per pair; zero
    //    padding rows K..Kp-1. Fast path u = h (Q_b rcp(gamma)) (Q_b is a power
    //    of two, so this is fl32(fl32(h Q_b) rcp(gamma))), which is within 1.5
    //    ulp of the exact quotient: unless u lies within |u| 2^-20 of a
    //    nonzero integer, no integer separates them and trunc(u) is the code.
    //    u is first clamped to +-(Q_b - 1/2): beyond that both give +-(Q_b - 1),
    //    so the extreme element needs no exact check (u = 0 needs none either).
    //    A lane with a near-integer u (rare) redoes all its codes exactly.
    //    For gamma below about Q_b / FLT_MAX (activations at subnormal scale)
    //    Q_b rcp(gamma) overflows and u means nothing: every lane then takes
    //    the exact division for all of its codes.
    const float cq = gamma != 0.0f ? qb * __builtin_amdgcn_rcpf(gamma) : 0.0f;
    const float ucl = qb - 0.5f;
    constexpr bool rn = kRne;
    int codes[NV][4];
    bool slow = !(cq <= 0x1.fffffep127f);
    if constexpr (!rn) {                               // truncation (the default): int(u) needs no clamp
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float h = (v[i][c] - mu32) * rs32;        // fl32(fl32(x - mu32) rs32)
                v[i][c] = h;
                const float u = __builtin_amdgcn_fmed3f(h * cq, -ucl, ucl);
                slow |= fabsf(u - rintf(u)) < fabsf(u) * 0x1p-20f;
                codes[i][c] = int(u);
            }
    } else {                                           // rounding: boundaries at half-integers
        const int qmax = int(qb) - 1;
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float h = (v[i][c] - mu32) * rs32;
                v[i][c] = h;
                const float u = __builtin_amdgcn_fmed3f(h * cq, -ucl, ucl);
                slow |= code_near_boundary(u, true);
                codes[i][c] = round_code(u, true, qmax);
            }
    }
    if (slow && gamma != 0.0f) {                       // gamma = 0: every h and code is 0
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) codes[i][c] = exact_code<rn>(v[i][c], qb, gamma, lim);
    }
    // sq: the thread's share of sum q (int8 form: every row; fp4 form: the
    // rows of types 0..2, whose 0/1 products need it)
    int sq = 0;
    if constexpr (kF4) {
        // octet (t, p) -> per digit c one dword at [tile t/4][p][c][word t%4]:
        // nibble n = digit c of |q| for row 32t + p + 4n, sign in bit 3. The
        // even rows' magnitudes sit in bytes of m0 (n = 0, 2, 4, 6), the odd
        // rows' in m1, so one shift and mask per half places a digit in
        // nibbles 2i and 2i + 1.
        uint32_t* q32 = reinterpret_cast<uint32_t*>(qs);
#pragma unroll
        for (int h = 0; h < NV / 2; ++h) {
            const int o = h * NT + tid;
            if (o >= octets) continue;
            const int t = o >> 2, p = o & 3;
            uint32_t m0 = 0, m1 = 0, sg = 0;
            int s8 = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int a = codes[2 * h][c], b = codes[2 * h + 1][c];
                m0 |= uint32_t(a < 0 ? -a : a) << (8 * c);
                m1 |= uint32_t(b < 0 ? -b : b) << (8 * c);
                sg |= uint32_t(a < 0) << (8 * c + 3) | uint32_t(b < 0) << (8 * c + 7);
                s8 += a + b;
            }
            sq += p != 3 ? s8 : 0;
            uint32_t* dst = q32 + (t >> 2) * 64 + p * 16 + (t & 3);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                dst[4 * c] = __builtin_amdgcn_bitop3_b32(m0 >> (2 * c), 0x03030303u,
                                                         ((m1 >> (2 * c)) & 0x03030303u) << 4 | sg, 0xEA);
            if (xq_opt && blockIdx.x == 0) {
                const int64_t k0 = 32 * t + p;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    xq_opt[k0 + 8 * c] = int8_t(codes[2 * h][c]);
                    xq_opt[k0 + 8 * c + 4] = int8_t(codes[2 * h + 1][c]);
                }
            }
        }
        // words K/32 .. 4 TQ - 1 (padding rows) and the zero tile
        const int w0 = int(K >> 5), nz = (4 * int(TQ) - w0) * 16;
        for (int z = tid; z < nz; z += NT) {
            const int t = w0 + (z >> 4);
            q32[(t >> 2) * 64 + (z & 15) * 4 + (t & 3)] = 0u;
        }
        if (tid < 64) q32[(kFusedMaxKp / 128) * 64 + tid] = 0u;
    } else {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int p = i * NT + tid;
            if (p >= pairs) continue;
            const uint32_t word = uint32_t(uint8_t(codes[i][0])) | uint32_t(uint8_t(codes[i][1])) << 8 |
                                  uint32_t(uint8_t(codes[i][2])) << 16 | uint32_t(uint8_t(codes[i][3])) << 24;
            sq += (codes[i][0] + codes[i][1]) + (codes[i][2] + codes[i][3]);
            const int t = p >> 3, sr = p & 7;
            *reinterpret_cast<uint32_t*>(qs + (t >> 2) * 128 + sr * 16 + (t & 3) * 4) = word;
            if (xq_opt && blockIdx.x == 0) {
                const int64_t k0 = 32 * t + sr;
#pragma unroll
                for (int c = 0; c < 4; ++c) xq_opt[k0 + 8 * c] = int8_t(codes[i][c]);
            }
        }
        for (int k = int(K) + tid; k < Kp; k += NT) qs[q_pos(k)] = 0;
        if (tid < 32) reinterpret_cast<uint32_t*>(qs + kFusedMaxKp)[tid] = 0u;
    }
    if (gamma_opt && blockIdx.x == 0 && tid == 0) gamma_opt[0] = gamma;
    sq = wave_sum63_i(sq);
    if (lane == 63) iscr[wave] = sq;
    __syncthreads();

    // 4. per column group: the product (int8 form: token 0 in the lanes with
    //    r == 0; fp4 form: its four digits in the lanes with r < 4), then the
    //    KQ parts' sums through LDS (one barrier per group; none when a wave
    //    covers all of K) and the epilogue
    int rowsum = 0;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) rowsum += iscr[wv];
    const float scale = (beta0 * gamma) / qb;
    // the B operand: lanes past the token's columns never load it, and whatever their registers
    // hold only reaches token columns that are never read (an empty asm
    // defines the registers without spending instructions on zeros)
    i32x4_t bk[8];
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) asm volatile("" : "=v"(bk[s8]));
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int64_t grp = int64_t(blockIdx.x) + int64_t(it) * gridDim.x;
        if (grp >= ngroups) break;
        i32x4_t sum;
        if constexpr (kF4) {
            // lanes r < 4 read digit r of the step's codes (16 bytes per
            // type); the other lanes' columns are never read, so their B
            // operand may hold anything (any nibble is a finite fp4 value)
            f32x4_t acc[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) acc[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < S; ++i) {
                const int st = kq + KQ * i, tq = st * 4 + g;
                const i32x4_t* src = reinterpret_cast<const i32x4_t*>(qs) +
                                     (st < steps && tq < int(TQ) ? tq : kFusedMaxKp / 128) * 16 + r;
                if (r < 4) {
#pragma unroll
                    for (int p = 0; p < 4; ++p) bk[p] = src[4 * p];
                }
                w1a8_f4_step(w[it][i], bk, acc);
            }
            sum = w1a8_f4_combine(acc, r);
        } else {
            i32x4_t acc[8], accn[kTern ? 8 : 1];
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8) acc[s8] = i32x4_t{0, 0, 0, 0};
            if constexpr (kTern) {
#pragma unroll
                for (int s8 = 0; s8 < 8; ++s8) accn[s8] = i32x4_t{0, 0, 0, 0};
            }
            // only lanes r == 0 (token 0) read the codes: the other lanes'
            // token columns are never read, so their B operand may hold
            // anything; steps past the column's tiles read the zero code
            // tile, which cancels their unmasked signs. Reading for 4 lanes
            // instead of 64 saves LDS return bandwidth.
#pragma unroll
            for (int i = 0; i < S; ++i) {
                const int st = kq + KQ * i, tq = st * 4 + g;
                const i32x4_t* src = reinterpret_cast<const i32x4_t*>(
                    qs + (st < steps && tq < int(TQ) ? tq : kFusedMaxKp / 128) * 128);
                if (r == 0) {
#pragma unroll
                    for (int s8 = 0; s8 < 8; ++s8) bk[s8] = src[s8];
                }
                w1a8_step(w[it][i], bk, acc);
                if constexpr (kTern) w1a8_step(wn[it][i], bk, accn);
            }
            sum = w1a8_combine(acc);
            if constexpr (kTern) sum -= w1a8_combine(accn);
        }
        if constexpr (KQ > 1) {
            red[it & 1][wave][lane] = sum;
            __syncthreads();
            if (kq != 0 || r != 0) continue;
#pragma unroll
            for (int q = 1; q < KQ; ++q) sum += red[it & 1][f + F * q][lane];
        } else {
            if (r != 0) continue;
        }
        const int64_t j0 = grp * 16 * F + 16 * f + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t col = j0 + i;
            if (col >= N) continue;
            // binary: 2 sum b q - sum q (fp4 form: sum over the rows of types 0..2 only)
            const int32_t a = kTern ? sum[i] : kF4 ? sum[i] - rowsum : 2 * sum[i] - rowsum;
            y[col] = float(a) * scale;
            if (acc_opt) acc_opt[col] = a;
        }
    }
}

bool w1a8_decode1_supported(int64_t K) { return padded_k(K) <= kFusedMaxKp; }

// The fragments per group F (a divisor of NW whose steps fit the tile budget)
// and the groups per block IT, for NV pieces per thread.
template <int NV, int NW, bool kTern>
constexpr bool w1a8_d1_ok(int f, int it) {
    return f <= NW && NW % f == 0 && it * w1a8_d1_steps(NV, f) * (kTern ? 2 : 1) <= kD1MaxTiles;
}

template <int NV, int NW, int F, typename XT, bool kTern>
static void launch_w1a8_decode1_f(int it, unsigned grid, const XT* x, int64_t K, int64_t N, int64_t TQ, double eps,
                                  float qb, float lim, int rne, const uint32_t* P, const float* beta, float* y,
                                  int32_t* acc_opt, int8_t* xq_opt, float* gamma_opt, hipStream_t s) {
    const double rk = 1.0 / double(K);
#define BGB_D1X(ITV)                                                                                             \
    if (rne)                                                                                                     \
        bitlinear_decode1_kernel<NV, NW, F, ITV, XT, true, kTern><<<grid, NW * 64, 0, s>>>(x, K, rk, N, TQ, eps, \
                                                                                          qb, lim, P, beta, y,  \
                                                                                          acc_opt, xq_opt,      \
                                                                                          gamma_opt);           \
    else                                                                                                         \
        bitlinear_decode1_kernel<NV, NW, F, ITV, XT, false, kTern><<<grid, NW * 64, 0, s>>>(x, K, rk, N, TQ, eps, \
                                                                                           qb, lim, P, beta, y, \
                                                                                           acc_opt, xq_opt,     \
                                                                                           gamma_opt)
    if constexpr (w1a8_d1_ok<NV, NW, kTern>(F, 1)) {
        if constexpr (w1a8_d1_ok<NV, NW, kTern>(F, 2)) {
            if (it == 2) {
                BGB_D1X(2);
                return;
            }
        }
        BGB_D1X(1);
    }
#undef BGB_D1X
}

template <int NV, int NW, typename XT, bool kTern>
static void launch_w1a8_decode1_nv(const XT* x, int64_t K, int64_t N, int64_t TQ, double eps, float qb, float lim,
                                   int rne, const uint32_t* P, const float* beta, float* y, int32_t* acc_opt,
                                   int8_t* xq_opt, float* gamma_opt, hipStream_t s) {
    // the fewest fragments per group that give each block (one per CU) a
    // single group; failing that, the most allowed and up to 2 groups per
    // block, then more blocks
    const int64_t frags = (N + 15) / 16;
    int F = 1;
    while (2 * F <= NW && w1a8_d1_ok<NV, NW, kTern>(2 * F, 1) && (frags + F - 1) / F > kD1MaxGrid) F *= 2;
    const int64_t groups = (frags + F - 1) / F;
    int64_t grid = groups < kD1MaxGrid ? groups : kD1MaxGrid;
    int it = int((groups + grid - 1) / grid);
    const int it_max = w1a8_d1_ok<NV, NW, kTern>(F, 2) ? 2 : 1;
    if (it > it_max) {
        it = it_max;
        grid = (groups + it - 1) / it;
    }
    const unsigned gr = unsigned(grid);
#define BGB_D1F(FV)                                                                                              \
    launch_w1a8_decode1_f<NV, NW, FV, XT, kTern>(it, gr, x, K, N, TQ, eps, qb, lim, rne, P, beta, y, acc_opt,    \
                                                 xq_opt, gamma_opt, s)
    if (F == 1) BGB_D1F(1);
    else if (F == 2) BGB_D1F(2);
    else if (F == 4) BGB_D1F(4);
    else BGB_D1F(8);
#undef BGB_D1F
}

template <int NW, typename XT, bool kTern>
static void launch_w1a8_decode1_nw(const XT* x, int64_t K, int64_t N, double eps, float qb, float lim, int rne,
                                   const uint32_t* P, const float* beta, float* y, int32_t* acc_opt, int8_t* xq_opt,
                                   float* gamma_opt, hipStream_t s) {
    constexpr int nt = NW * 64;
    constexpr int kMaxNv = kFusedMaxKp / (nt * 4);     // 16 for 4 waves, 8 for 8
    const int64_t TQ = tiles_per_col(K);
    const int nv = int((TQ * 128 + nt * 4 - 1) / (nt * 4));
    const int nvp = nv <= 1 ? 1 : nv <= 2 ? 2 : nv <= 4 ? 4 : nv <= 8 ? 8 : 16;
#define BGB_D1(NVV)                                                                                              \
    launch_w1a8_decode1_nv<NVV, NW, XT, kTern>(x, K, N, TQ, eps, qb, lim, rne, P, beta, y, acc_opt, xq_opt,      \
                                               gamma_opt, s)
    if (nvp == 1) BGB_D1(1);
    else if (nvp == 2) BGB_D1(2);
    else if (nvp == 4) BGB_D1(4);
    else if (nvp == 8) BGB_D1(8);
    else if constexpr (kMaxNv >= 16 && !kTern) BGB_D1(16);   // ternary takes 8-wave blocks there
#undef BGB_D1
}

template <bool kTern>
static void launch_w1a8_decode1_t(const void* x, int x_bf16, int64_t K, int64_t N, double eps, float qb, float lim,
                                  int rne, const uint32_t* P, const float* beta, float* y, int32_t* acc_opt,
                                  int8_t* xq_opt, float* gamma_opt, hipStream_t s) {
    // 8-wave blocks for layers of at least 8192 columns; 4-wave blocks (one
    // wave per SIMD, so the per-wave prologue work is not repeated) below.
    // Ternary weights take two tiles per step, so K > 8192 (16 code dwords
    // per thread of a 4-wave block) also goes to 8-wave blocks.
    const bool wide = (N + 31) / 32 >= kD1MaxGrid || (kTern && padded_k(K) > 8192);
    if (x_bf16) {
        const uint16_t* xb = static_cast<const uint16_t*>(x);
        if (wide) launch_w1a8_decode1_nw<8, uint16_t, kTern>(xb, K, N, eps, qb, lim, rne, P, beta, y, acc_opt, xq_opt,
                                                             gamma_opt, s);
        else launch_w1a8_decode1_nw<4, uint16_t, kTern>(xb, K, N, eps, qb, lim, rne, P, beta, y, acc_opt, xq_opt,
                                                        gamma_opt, s);
    } else {
        const float* xf = static_cast<const float*>(x);
        if (wide) launch_w1a8_decode1_nw<8, float, kTern>(xf, K, N, eps, qb, lim, rne, P, beta, y, acc_opt, xq_opt,
                                                          gamma_opt, s);
        else launch_w1a8_decode1_nw<4, float, kTern>(xf, K, N, eps, qb, lim, rne, P, beta, y, acc_opt, xq_opt,
                                                     gamma_opt, s);
    }
}

hipError_t launch_w1a8_decode1(const void* x, int x_bf16, int64_t K, int64_t N, double eps, float qb, float lim,
                               int rne, const uint32_t* P, const float* beta, float* y, int32_t* acc_opt, int8_t* xq_opt,
                               float* gamma_opt, int tern, hipStream_t s) {
    if (tern) launch_w1a8_decode1_t<true>(x, x_bf16, K, N, eps, qb, lim, rne, P, beta, y, acc_opt, xq_opt, gamma_opt, s);
    else launch_w1a8_decode1_t<false>(x, x_bf16, K, N, eps, qb, lim, rne, P, beta, y, acc_opt, xq_opt, gamma_opt, s);
    return hipGetLastError();
}

hipError_t launch_w1a8_gemv(const int8_t* q, const int32_t* rowsum, const float* gamma, int gstride,
                            const float* beta, float qb, int64_t M, int64_t K, int64_t N, const uint32_t* P, float* y,
                            int32_t* acc_opt, int tern, hipStream_t s) {
    const unsigned grid = unsigned((N + 15) / 16);
    const int64_t TQ = tiles_per_col(K);
    const int tf = int((M + 15) / 16);
    int gs = gen_steps(TQ);
    if (tern && gs > 2) gs = 2;      // two sign planes: fewer steps per pass keep the registers in bounds
    constexpr unsigned nt = kGenWaves * 64;
#define BGB_G8(TFV, GSV)                                                                                          \
    if (tern) gemv_w1a8_kernel<TFV, GSV, true><<<grid, nt, 0, s>>>(q, rowsum, gamma, gstride, beta, qb, int(M), N, TQ, \
                                                                   P, y, acc_opt);                               \
    else gemv_w1a8_kernel<TFV, GSV, false><<<grid, nt, 0, s>>>(q, rowsum, gamma, gstride, beta, qb, int(M), N, TQ, \
                                                                P, y, acc_opt)
#define BGB_G8S(TFV)                                                                                              \
    if (gs == 1) { BGB_G8(TFV, 1); } else if (gs == 2) { BGB_G8(TFV, 2); }                                      \
    else { gemv_w1a8_kernel<TFV, 4, false><<<grid, nt, 0, s>>>(q, rowsum, gamma, gstride, beta, qb, int(M), N, TQ, \
                                                                 P, y, acc_opt); }
    if (tf == 1) { BGB_G8S(1) } else { BGB_G8S(2) }       // M <= 32: at most two token fragments
#undef BGB_G8S
#undef BGB_G8
    return hipGetLastError();
}

// ----------------------------------------------------------------- W1A16 -----

// Field-bit constants per 16-bit format: P0 = first field bit used; the 1.0
// and 0.5 bases replicated in both halves of a dword.
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

// A operand of MFMA u: the four words' bit pair (u, u+16) moved to field bit p.
template <bool kF16, int U>
BGB_DEV u32x4_t w1a16_a(const u32x4_t& w) {
    using F = Fmt16<kF16>;
    constexpr int T = U % 4;
    constexpr int p = F::P0 + T;
    constexpr int sh = p - U;
    constexpr uint32_t mask = 0x00010001u << p;
    constexpr uint32_t base = (T == 3) ? F::kHalf : F::kOne;
    u32x4_t a;   // (shifted & mask) | base as one bitop3 (truth table 0xEA); the 4 shifts are shared by 4 U
    a.x = __builtin_amdgcn_bitop3_b32(shift_word<sh>(w.x), mask, base, 0xEA);
    a.y = __builtin_amdgcn_bitop3_b32(shift_word<sh>(w.y), mask, base, 0xEA);
    a.z = __builtin_amdgcn_bitop3_b32(shift_word<sh>(w.z), mask, base, 0xEA);
    a.w = __builtin_amdgcn_bitop3_b32(shift_word<sh>(w.w), mask, base, 0xEA);
    return a;
}

// One step (16 MFMAs) for TF token fragments; b(u, tf) yields the B operand.
template <bool kF16, int TF, int U, typename BF>
BGB_DEV void w1a16_u(const u32x4_t& w, BF&& bsrc, f32x4_t (*acc)[4]) {
    const u32x4_t a = w1a16_a<kF16, U>(w);
#pragma unroll
    for (int tf = 0; tf < TF; ++tf) acc[tf][U % 4] = mfma16<kF16>(a, bsrc(U, tf), acc[tf][U % 4]);
}
template <bool kF16, int TF, typename BF>
BGB_DEV void w1a16_step(const u32x4_t& w, BF&& bsrc, f32x4_t (*acc)[4]) {
    w1a16_u<kF16, TF, 0>(w, bsrc, acc);  w1a16_u<kF16, TF, 1>(w, bsrc, acc);
    w1a16_u<kF16, TF, 2>(w, bsrc, acc);  w1a16_u<kF16, TF, 3>(w, bsrc, acc);
    w1a16_u<kF16, TF, 4>(w, bsrc, acc);  w1a16_u<kF16, TF, 5>(w, bsrc, acc);
    w1a16_u<kF16, TF, 6>(w, bsrc, acc);  w1a16_u<kF16, TF, 7>(w, bsrc, acc);
    w1a16_u<kF16, TF, 8>(w, bsrc, acc);  w1a16_u<kF16, TF, 9>(w, bsrc, acc);
    w1a16_u<kF16, TF, 10>(w, bsrc, acc); w1a16_u<kF16, TF, 11>(w, bsrc, acc);
    w1a16_u<kF16, TF, 12>(w, bsrc, acc); w1a16_u<kF16, TF, 13>(w, bsrc, acc);
    w1a16_u<kF16, TF, 14>(w, bsrc, acc); w1a16_u<kF16, TF, 15>(w, bsrc, acc);
}

// All 16 A operands of a step (64 registers), for reuse across token fragments.
template <bool kF16>
BGB_DEV void w1a16_decode(const u32x4_t& w, u32x4_t* a) {
    a[0] = w1a16_a<kF16, 0>(w);   a[1] = w1a16_a<kF16, 1>(w);   a[2] = w1a16_a<kF16, 2>(w);
    a[3] = w1a16_a<kF16, 3>(w);   a[4] = w1a16_a<kF16, 4>(w);   a[5] = w1a16_a<kF16, 5>(w);
    a[6] = w1a16_a<kF16, 6>(w);   a[7] = w1a16_a<kF16, 7>(w);   a[8] = w1a16_a<kF16, 8>(w);
    a[9] = w1a16_a<kF16, 9>(w);   a[10] = w1a16_a<kF16, 10>(w); a[11] = w1a16_a<kF16, 11>(w);
    a[12] = w1a16_a<kF16, 12>(w); a[13] = w1a16_a<kF16, 13>(w); a[14] = w1a16_a<kF16, 14>(w);
    a[15] = w1a16_a<kF16, 15>(w);
}

// Output for one token: s = 2 sum_k b x - sum_k x from the type accumulators.
BGB_DEV float w1a16_out(const f32x4_t* tot, int i, float X0, float X1, float X2, float X3) {
    const float sb = ((8.0f * (tot[0][i] - X0) + 4.0f * (tot[1][i] - X1)) + 2.0f * (tot[2][i] - X2)) +
                     2.0f * (tot[3][i] - 0.5f * X3);
    return 2.0f * sb - (((X0 + X1) + X2) + X3);
}

// Single token on the fp4 x fp8 matrix cores (16 x 16 x 128, fp8 = e4m3).
// A holds the signs as fp4 +-1.0: MFMA type p (0..3) takes bit 4n + p of word
// d of the lane's tile into nibble n of dword d (tile row 32d + 4n + p), moved
// to the sign field of 1.0 (a set bit gives +1). B holds the token scaled by
// 2^sc (its largest magnitude then lies in [8, 16)) as five fixed-point limbs
// in token columns 0..4, each an integer in [-16, 16]: l0 = rint(v), then
// l_c = rint(16 r_c) with r_1 = v - l0 and r_(c+1) = 16 r_c - l_c (every step
// exact in fp32), so v = l0 + l1/16 + l2/256 + l3/4096 + l4/65536 up to at
// most 2^-17 (exact whenever v is a multiple of 2^-16: a bf16 value within
// 2^-12 of the largest magnitude, and every integer while the largest
// magnitude is below 2^20). The matrix cores align
// a column's 128 products to the largest one and keep about 14 bits below it
// (measured: fp8 values more than 2^13 below the largest in their column are
// dropped), so every limb column must hold values of one quantum; integers
// below 2^5 are, and each column's sums stay exact integers. The lane layout
// pairs fp4 lane group ga's nibbles 16h + u with fp8 lane group
// (2 ga + h) mod 4, byte 16 (ga / 2) + u (measured with one-element operands), so fp8 lane
// group gb reads rows of tiles 4 st + gb / 2 (bytes 0..15) and
// 4 st + 2 + gb / 2 (bytes 16..31), words 2 (gb % 2) and 2 (gb % 2) + 1.
// LDS: per 128-row tile and type p, per limb c, the 4 words' 8 rows each as
// bytes at f8_off(tile, p, c, word) + n; tile TQ is a zero tile. A token with
// an inf or NaN gives NaN outputs.
constexpr int kF8Limbs = 5;
constexpr int kF8TileBytes = 4 * kF8Limbs * 32;
constexpr int kF8LdsBytes = (kFusedMaxKp / 128 + 1) * kF8TileBytes;    // the largest K and the zero tile
constexpr int kF8GroupLds = 65536;                                      // the grouped kernel's dynamic LDS cap
BGB_DEV int f8_off(int tq, int p, int c, int d) { return ((tq * 4 + p) * kF8Limbs + c) * 32 + d * 8; }
template <int P>
BGB_DEV i32x4_t f4_pm1(const u32x4_t& w) {      // (~(w << (3 - P)) & 0x88888888) | 0x22222222
    constexpr int sh = 3 - P;
    return i32x4_t{int(__builtin_amdgcn_bitop3_b32(w.x << sh, 0x88888888u, 0x22222222u, 0xAE)),
                   int(__builtin_amdgcn_bitop3_b32(w.y << sh, 0x88888888u, 0x22222222u, 0xAE)),
                   int(__builtin_amdgcn_bitop3_b32(w.z << sh, 0x88888888u, 0x22222222u, 0xAE)),
                   int(__builtin_amdgcn_bitop3_b32(w.w << sh, 0x88888888u, 0x22222222u, 0xAE))};
}
BGB_DEV f32x4_t mfma_f4f8(const i32x4_t& a, const i32x8_t& b, const f32x4_t& c) {
    const i32x8_t a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};   // fp4 A uses the first four dwords
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c, 4, 0, 0, 127, 0, 127);   // scales 2^0
}
// The limbs of 8 scaled values (|v| < 16), stored as 8 bytes each at dst + c * 32.
BGB_DEV void f8_limbs(float (&v)[8], uint8_t* dst) {
#pragma unroll
    for (int c = 0; c < kF8Limbs; ++c) {
        float t[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            t[n] = __builtin_rintf(v[n]);
            v[n] = 16.0f * (v[n] - t[n]);
        }
        int lo = 0, hi = 0;   // integers up to 16 in magnitude: exact in e4m3
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], lo, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], lo, true);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(t[4], t[5], hi, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(t[6], t[7], hi, true);
        *reinterpret_cast<uint2*>(dst + c * 32) = uint2{uint32_t(lo), uint32_t(hi)};
    }
}

// Single token, activation staging fused: the block scales the token and
// writes its limbs to LDS, once, then takes up to IT column groups
// (bid + i * nblk) of F 16-column fragments, as the W1A8 kernel. The body is
// shared by the one-linear kernel (bid, nblk = the block index and count)
// and the grouped one (the block's rank and count within its linear). LDS:
// xb [(TQ + 1) kF8TileBytes] (the limbs and a zero tile, the B operand of
// steps past the last tile), red [2 NW 64] when KQ > 1 (the K parts' sums),
// mx [NW].
template <bool kF16, int NV, int NW, int F, int IT>
BGB_DEV void fbi_decode1_body(const uint16_t* __restrict__ x, int64_t K, int64_t N, int64_t TQ,
                              const uint32_t* __restrict__ P, const void* __restrict__ alpha, int alpha_f16,
                              void* __restrict__ y, int y_dtype, int64_t bid, int64_t nblk, uint8_t* xb,
                              f32x4_t* red, uint32_t* mx) {
    constexpr int NT = NW * 64;
    constexpr int KQ = NW / F;
    constexpr int S = NV * F;          // steps per wave: TQ <= NV NT / 16 tiles = NV NW steps, over KQ waves
    static_assert(NW % F == 0 && IT * S <= kD1MaxTiles, "single-token W1A16 shape");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r = lane & 15, f = wave % F, kq = wave / F;
    const int64_t ngroups = (N + 16 * F - 1) / (16 * F);
    const int octets = int(K / 8), poct = int(TQ * 16);   // octets inside K; of the padded rows
    const int64_t steps = (TQ + 3) / 4;

    // 1. the token: octet o = (t, p) = (o / 4, o % 4) holds rows 32t + p + 4n,
    //    n = 0..7 (K % 32 == 0: an octet is all inside K or all padding, whose
    //    values are zero); the loads complete before the sign stream starts
    uint32_t xv[NV][4];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int o = i * NT + tid;
        const bool ok = o < octets;
        const uint16_t* xo = x + (ok ? 32 * (o >> 2) + (o & 3) : 0);
        const uint32_t keep = 0u - uint32_t(ok);
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[i][j] = (uint32_t(xo[8 * j]) | uint32_t(xo[8 * j + 4]) << 16) & keep;
    }
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));     // vmcnt(0): the token is in
    // the epilogue's arguments (on a later cache line of the argument block
    // than the first ones) pinned in registers from here on, so that they are
    // requested with the first ones; left alone, the compiler loads them after
    // the last product, in front of the stores
    asm volatile("" ::"s"(y), "s"(y_dtype), "s"(alpha_f16));
    u32x4_t w[IT][S];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int64_t grp = bid + int64_t(it) * nblk;
        const int64_t jj = grp < ngroups ? grp * 16 * F + 16 * f + r : N;
        preload<S>(w[it], P, kq, KQ, steps, TQ, N, jj, g);
    }
    // With one group per block, the scales of the 4 columns j0..j0+3 this
    // lane writes are requested here, behind the sign tiles the epilogue
    // waits for anyway, rather than after the last barrier (with several
    // groups, measured slower: the epilogue lanes are read late instead, while
    // the next group's tiles stream). Two 8-byte words: bytes 4 j0 and
    // 4 j0 + 8 for fp32, byte 2 j0 twice for fp16. j0 is a multiple of 4 and
    // alpha is 16-byte aligned, so a read past the N-th scale stays inside
    // the aligned 16 bytes holding scale j0; a group past N reads scale 0.
    constexpr bool kAlphaAhead = IT == 1;
    uint2 araw[2] = {};
    if constexpr (kAlphaAhead) {
        int64_t j0 = bid * 16 * F + 16 * f + 4 * g;
        j0 = j0 < N ? j0 : 0;
        const char* a8 = static_cast<const char*>(alpha);
        const int64_t lo = alpha_f16 ? 2 * j0 : 4 * j0, hi = alpha_f16 ? 2 * j0 : 4 * j0 + 8;
        araw[0] = *reinterpret_cast<const uint2*>(a8 + lo);
        araw[1] = *reinterpret_cast<const uint2*>(a8 + hi);
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. the largest magnitude (16-bit magnitude patterns order as the
    //    values; NaN above inf) and the scale 2^sc that puts it in [128, 256)
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) m = max(m, max(xv[i][j] & 0x7fffu, (xv[i][j] >> 16) & 0x7fffu));
    m = wave_umax63(m);
    if (lane == 63) mx[wave] = m;
    __syncthreads();
    uint32_t mt = mx[0];
#pragma unroll
    for (int wv = 1; wv < NW; ++wv) mt = max(mt, mx[wv]);
    const bool finite = mt < (kF16 ? 0x7c00u : 0x7f80u);
    const float xmax = kF16 ? f16_to_f32(uint16_t(mt)) : bf16_to_f32(uint16_t(mt));
    const int sc = finite && mt != 0 ? 4 - __builtin_amdgcn_frexp_expf(xmax) : 0;

    // 3. the limbs into LDS (padding octets store zeros), and the zero tile
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int o = i * NT + tid;
        if (o >= poct) continue;
        const int t = o >> 2, p = o & 3;
        float v[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint16_t e0 = uint16_t(xv[i][j] & 0xffffu), e1 = uint16_t(xv[i][j] >> 16);
            v[2 * j] = __builtin_amdgcn_ldexpf(kF16 ? f16_to_f32(e0) : bf16_to_f32(e0), sc);
            v[2 * j + 1] = __builtin_amdgcn_ldexpf(kF16 ? f16_to_f32(e1) : bf16_to_f32(e1), sc);
        }
        f8_limbs(v, xb + f8_off(t >> 2, p, 0, t & 3));      // xv[i][j] holds rows n = 2j, 2j + 1
    }
    const int kZeroTile = int(TQ);
    for (int z = tid; z < kF8TileBytes / 4; z += NT) reinterpret_cast<uint32_t*>(xb + kZeroTile * kF8TileBytes)[z] = 0u;
    __syncthreads();

    // 4. per column group: the product (the limbs live in lanes r < 5; the
    //    other lanes' B registers stay zero, since an undefined fp8 byte may
    //    be a NaN; tiles past the last one read the zero limb tile, since a
    //    zero sign word decodes to -1 weights), then the KQ parts' sums
    //    through LDS (none when a wave covers all of K)
    i32x8_t bq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) bq[q] = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int64_t grp = bid + int64_t(it) * nblk;
        if (grp >= ngroups) break;
        f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const int64_t st = kq + int64_t(KQ) * i;
            const int64_t ta = st * 4 + (g >> 1), tb = ta + 2;
            const bool oka = st < steps && ta < TQ, okb = st < steps && tb < TQ;
            const int c = r < kF8Limbs ? r : 0;
            const uint8_t* pa = xb + f8_off(oka ? int(ta) : kZeroTile, 0, c, 2 * (g & 1));
            const uint8_t* pb = xb + f8_off(okb ? int(tb) : kZeroTile, 0, c, 2 * (g & 1));
            if (r < kF8Limbs) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const i32x4_t ha = *reinterpret_cast<const i32x4_t*>(pa + kF8Limbs * 32 * q);
                    const i32x4_t hb = *reinterpret_cast<const i32x4_t*>(pb + kF8Limbs * 32 * q);
                    bq[q] = i32x8_t{ha.x, ha.y, ha.z, ha.w, hb.x, hb.y, hb.z, hb.w};
                }
            }
            const u32x4_t& wt = w[it][i];
            acc[0] = mfma_f4f8(f4_pm1<0>(wt), bq[0], acc[0]);
            acc[1] = mfma_f4f8(f4_pm1<1>(wt), bq[1], acc[1]);
            acc[0] = mfma_f4f8(f4_pm1<2>(wt), bq[2], acc[0]);
            acc[1] = mfma_f4f8(f4_pm1<3>(wt), bq[3], acc[1]);
        }
        // limb columns 0..4 weighted 16^-c, summed over the two quads of
        // lanes 0..7 of each row (the total lands in lane r = 0)
        f32x4_t z = acc[0] + acc[1];
        const float lw = __builtin_amdgcn_ldexpf(1.0f, -4 * r);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = r < kF8Limbs ? z[e] * lw : 0.0f;
            v += dpp_f32<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
            v += dpp_f32<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
            v += dpp_f32<0x104, 0xF>(v);  // row_shl:4 (lane r + 4; zero past the row)
            z[e] = v;
        }
        if constexpr (KQ > 1) {
            red[((it & 1) * NW + wave) * 64 + lane] = z;
            __syncthreads();
            if (kq != 0 || r != 0) continue;
            // the parts in a fixed order: kq = 0, 1, ..., KQ - 1
#pragma unroll
            for (int q = 1; q < KQ; ++q) z += red[((it & 1) * NW + f + F * q) * 64 + lane];
        } else {
            if (r != 0) continue;
        }
        const int64_t j0 = grp * 16 * F + 16 * f + 4 * g;
        const uint32_t aw[4] = {araw[0].x, araw[0].y, araw[1].x, araw[1].y};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t col = j0 + i;
            if (col >= N) continue;
            const float a = !kAlphaAhead ? load_alpha(alpha, alpha_f16, col)
                            : alpha_f16  ? f16_to_f32(uint16_t(aw[i >> 1] >> (16 * (i & 1))))
                                         : __uint_as_float(aw[i]);
            const float s = finite ? __builtin_amdgcn_ldexpf(z[i], -sc) : __builtin_nanf("");
            store_y(y, y_dtype, col, a * s);
        }
    }
}

template <bool kF16, int NV, int NW, int F, int IT>
__global__ void __launch_bounds__(NW * 64)
fbi_decode1_kernel(const uint16_t* __restrict__ x, int64_t K, int64_t N, int64_t TQ, const uint32_t* __restrict__ P,
                   const void* __restrict__ alpha, int alpha_f16, void* __restrict__ y, int y_dtype) {
    constexpr int KQ = NW / F;
    __shared__ __attribute__((aligned(16))) uint8_t xb[kF8LdsBytes];
    __shared__ f32x4_t red[(KQ > 1 ? 2 * NW : 1) * 64];
    __shared__ uint32_t mx[NW];
    fbi_decode1_body<kF16, NV, NW, F, IT>(x, K, N, TQ, P, alpha, alpha_f16, y, y_dtype, blockIdx.x, gridDim.x, xb,
                                          red, mx);
}

bool w1a16_decode1_supported(int64_t K) { return padded_k(K) <= kFusedMaxKp; }

template <int NV, int NW>
constexpr bool w1a16_d1_ok(int f, int it) {
    return f <= NW && NW % f == 0 && it * NV * f <= kD1MaxTiles;
}

template <bool kF16, int NV, int NW, int F>
static void launch_w1a16_decode1_f(int it, unsigned grid, const uint16_t* x, int64_t K, int64_t N, int64_t TQ,
                                   const uint32_t* P, const void* alpha, int alpha_f16, void* y, int y_dtype,
                                   hipStream_t s) {
#define BGB_F1X(ITV) \
    fbi_decode1_kernel<kF16, NV, NW, F, ITV><<<grid, NW * 64, 0, s>>>(x, K, N, TQ, P, alpha, alpha_f16, y, y_dtype)
    if constexpr (w1a16_d1_ok<NV, NW>(F, 1)) {
        if constexpr (w1a16_d1_ok<NV, NW>(F, 2)) {
            if (it == 2) {
                BGB_F1X(2);
                return;
            }
        }
        BGB_F1X(1);
    }
#undef BGB_F1X
}

template <bool kF16, int NV, int NW>
static void launch_w1a16_decode1_nv(const uint16_t* x, int64_t K, int64_t N, int64_t TQ, const uint32_t* P,
                                    const void* alpha, int alpha_f16, void* y, int y_dtype, hipStream_t s) {
    // as for W1A8: the fewest fragments per group that give each block one
    // group, else the most allowed and up to 2 groups per block
    const int64_t frags = (N + 15) / 16;
    int F = 1;
    while (2 * F <= NW && w1a16_d1_ok<NV, NW>(2 * F, 1) && (frags + F - 1) / F > kD1MaxGrid) F *= 2;
    const int64_t groups = (frags + F - 1) / F;
    int64_t grid = groups < kD1MaxGrid ? groups : kD1MaxGrid;
    int it = int((groups + grid - 1) / grid);
    const int it_max = w1a16_d1_ok<NV, NW>(F, 2) ? 2 : 1;
    if (it > it_max) {
        it = it_max;
        grid = (groups + it - 1) / it;
    }
    const unsigned gr = unsigned(grid);
#define BGB_F1F(FV) launch_w1a16_decode1_f<kF16, NV, NW, FV>(it, gr, x, K, N, TQ, P, alpha, alpha_f16, y, y_dtype, s)
    if (F == 1) BGB_F1F(1);
    else if (F == 2) BGB_F1F(2);
    else if (F == 4) BGB_F1F(4);
    else BGB_F1F(8);
#undef BGB_F1F
}

template <bool kF16, int NW>
static void launch_w1a16_decode1_nw(const uint16_t* x, int64_t K, int64_t N, const uint32_t* P, const void* alpha,
                                    int alpha_f16, void* y, int y_dtype, hipStream_t s) {
    constexpr int nt = NW * 64;
    constexpr int kMaxNv = kFusedMaxKp / (nt * 8);     // 16-byte pieces per thread: 8 for 4 waves, 4 for 8
    const int64_t TQ = tiles_per_col(K);
    const int nv = int((TQ * 16 + nt - 1) / nt);
    const int nvp = nv <= 1 ? 1 : nv <= 2 ? 2 : nv <= 4 ? 4 : 8;
#define BGB_F1(NVV) launch_w1a16_decode1_nv<kF16, NVV, NW>(x, K, N, TQ, P, alpha, alpha_f16, y, y_dtype, s)
    if (nvp == 1) BGB_F1(1);
    else if (nvp == 2) BGB_F1(2);
    else if (nvp == 4) BGB_F1(4);
    else if constexpr (kMaxNv >= 8) BGB_F1(8);
#undef BGB_F1
}

hipError_t launch_w1a16_decode1(const void* x, int x_f16, int64_t K, int64_t N, const uint32_t* P,
                                const void* alpha, int alpha_f16, void* y, int y_dtype, hipStream_t s) {
    // 8-wave blocks for layers of at least 8192 columns, 4-wave blocks below
    const uint16_t* xx = static_cast<const uint16_t*>(x);
    const bool wide = (N + 31) / 32 >= kD1MaxGrid;
    if (x_f16) {
        if (wide) launch_w1a16_decode1_nw<true, kD1Waves>(xx, K, N, P, alpha, alpha_f16, y, y_dtype, s);
        else launch_w1a16_decode1_nw<true, 4>(xx, K, N, P, alpha, alpha_f16, y, y_dtype, s);
    } else {
        if (wide) launch_w1a16_decode1_nw<false, kD1Waves>(xx, K, N, P, alpha, alpha_f16, y, y_dtype, s);
        else launch_w1a16_decode1_nw<false, 4>(xx, K, N, P, alpha, alpha_f16, y, y_dtype, s);
    }
    return hipGetLastError();
}

// Several independent single-token linears in one launch. Each linear is
// split into column groups of F fragments with 8-wave blocks, one group per
// block: the fewest fragments per group that give at most one block per CU,
// within at most kGroupSteps sign tiles per thread (the shapes that need
// about 100 VGPRs, so that two blocks share a CU; the larger shapes of the
// one-linear kernel would leave one block per CU). The grid is the concatenation of the linears' blocks,
// those with the most sign bytes per block first. A block finds its linear
// from the table in the kernel arguments (uniform selects, no indexing) and
// runs the same body as the one-linear kernel. Measured on the four linears
// of a 7B-shaped layer (25.5 MB of signs): 17.5-18 us against 26.5 us for
// four launches; reading the activations only in the lanes that use them
// (as the one-linear kernel does for 8 steps) or larger blocks were slower.
constexpr int kGroupSteps = 4;
struct D1Item {
    const uint16_t* x;
    const uint32_t* P;
    const void* alpha;
    void* y;
    int64_t K, N, TQ;
    int first, nblk, cfg;   // first block, block count, (NV, F) case
};
struct D1Group {
    D1Item it[kGroupMax];
    int count, alpha_f16, y_dtype;
};

template <bool kF16>
__global__ void __launch_bounds__(kD1Waves * 64)
fbi_decode1_group_kernel(const D1Group g) {
    constexpr int NW = kD1Waves;
    extern __shared__ __attribute__((aligned(16))) uint8_t xb_dyn[];   // (largest TQ + 1) tiles of limbs
    uint8_t* xb = xb_dyn;
    __shared__ f32x4_t red[2 * NW * 64];
    __shared__ uint32_t mx[NW];
    D1Item it = g.it[0];
#pragma unroll
    for (int i = 1; i < kGroupMax; ++i)
        if (i < g.count && int(blockIdx.x) >= g.it[i].first) it = g.it[i];
    const int64_t bid = int64_t(blockIdx.x) - it.first;
#define BGB_G1(C, NVV, FV, ITV)                                                                                 \
    case C:                                                                                                  \
        fbi_decode1_body<kF16, NVV, NW, FV, ITV>(it.x, it.K, it.N, it.TQ, it.P, it.alpha, g.alpha_f16, it.y,  \
                                                 g.y_dtype, bid, it.nblk, xb, red, mx);                       \
        break;
    static_assert(kGroupSteps == 4, "the cases below are the shapes with NV F <= 4");
    switch (it.cfg) {
        BGB_G1(0, 1, 1, 1)
        BGB_G1(1, 1, 2, 1)
        BGB_G1(2, 1, 4, 1)
        BGB_G1(3, 2, 1, 1)
        BGB_G1(4, 2, 2, 1)
        BGB_G1(5, 4, 1, 1)
        BGB_G1(6, 1, 4, 2)
        BGB_G1(7, 2, 2, 2)
        BGB_G1(8, 4, 1, 2)
        default: break;
    }
#undef BGB_G1
}

// A grouped block holds its linear's limbs in dynamic LDS, at most
// kF8GroupLds bytes so that two blocks share a CU: K up to 12928.
bool w1a16_decode1_group_item_ok(int64_t K) {
    return w1a16_decode1_supported(K) && (tiles_per_col(K) + 1) * kF8TileBytes <= kF8GroupLds;
}

bool w1a16_decode1_group_supported(const W1a16Item* items, int count) {
    if (count < 0 || count > kGroupMax) return false;
    for (int i = 0; i < count; ++i)
        if (!w1a16_decode1_group_item_ok(items[i].K)) return false;
    return true;
}

hipError_t launch_w1a16_decode1_group(const W1a16Item* items, int count, int x_f16, int alpha_f16, int y_dtype,
                                      hipStream_t s) {
    if (!w1a16_decode1_group_supported(items, count)) return hipErrorInvalidValue;
    constexpr int NW = kD1Waves, NT = NW * 64;
    D1Group g{};
    int order[kGroupMax], n = 0;
    int nvps[kGroupMax], Fs[kGroupMax], ITs[kGroupMax];
    int64_t frag[kGroupMax], cost[kGroupMax];
    auto blocks = [&](int i) { return ((frag[i] + Fs[i] - 1) / Fs[i] + ITs[i] - 1) / ITs[i]; };
    int64_t total_blocks = 0;
    for (int i = 0; i < count; ++i) {
        if (items[i].N <= 0) continue;                   // an empty linear takes no blocks
        const W1a16Item& in = items[i];
        D1Item& d = g.it[n];
        d.x = static_cast<const uint16_t*>(in.x);
        d.P = in.P;
        d.alpha = in.alpha;
        d.y = in.y;
        d.K = in.K;
        d.N = in.N;
        d.TQ = tiles_per_col(in.K);
        const int nv = int((d.TQ * 16 + NT - 1) / NT);
        nvps[n] = nv <= 1 ? 1 : nv <= 2 ? 2 : 4;
        frag[n] = (in.N + 15) / 16;
        int F = 1;                                       // enough blocks for the linear alone to fill the chip
        while (nvps[n] * 2 * F <= kGroupSteps && (frag[n] + F - 1) / F > kD1MaxGrid) F *= 2;
        Fs[n] = F;
        ITs[n] = 1;
        total_blocks += blocks(n);
        order[n] = n;
        ++n;
    }
    // Every block stages its token and sums it before any product, so more
    // blocks than the chip holds at once (two per CU) repeat that prologue in
    // later rounds. Coarsen the linear with the most blocks (more fragments
    // per group, then two groups per block) until they fit or none can grow.
    while (total_blocks > 2 * kD1MaxGrid) {
        int best = -1;
        for (int i = 0; i < n; ++i) {
            const bool grow = nvps[i] * Fs[i] * 2 <= kGroupSteps || ITs[i] == 1;
            if (grow && (best < 0 || blocks(i) > blocks(best))) best = i;
        }
        if (best < 0) break;
        total_blocks -= blocks(best);
        if (nvps[best] * Fs[best] * 2 <= kGroupSteps) Fs[best] *= 2;
        else ITs[best] = 2;
        total_blocks += blocks(best);
    }
    for (int i = 0; i < n; ++i) {
        D1Item& d = g.it[i];
        const int F = Fs[i], nvp = nvps[i];
        d.nblk = int(blocks(i));
        if (ITs[i] == 1) d.cfg = nvp == 1 ? (F == 1 ? 0 : F == 2 ? 1 : 2) : nvp == 2 ? (F == 1 ? 3 : 4) : 5;
        else d.cfg = nvp == 1 ? 6 : nvp == 2 ? 7 : 8;     // F = kGroupSteps / nvp, two groups per block
        cost[i] = int64_t(F) * ITs[i] * d.TQ;
    }
    if (n == 0) return hipSuccess;
    // heaviest blocks first (stable), then the prefix sums of the block counts
    for (int a = 1; a < n; ++a)
        for (int b = a; b > 0 && cost[order[b]] > cost[order[b - 1]]; --b) {
            const int t = order[b];
            order[b] = order[b - 1];
            order[b - 1] = t;
        }
    D1Group h{};
    int64_t total = 0;
    for (int i = 0; i < n; ++i) {
        h.it[i] = g.it[order[i]];
        h.it[i].first = int(total);
        total += h.it[i].nblk;
    }
    h.count = n;
    h.alpha_f16 = alpha_f16;
    int64_t tq_max = 0;
    for (int i = 0; i < n; ++i) tq_max = h.it[i].TQ > tq_max ? h.it[i].TQ : tq_max;
    const size_t lds = size_t(tq_max + 1) * kF8TileBytes;
    h.y_dtype = y_dtype;
    if (x_f16) fbi_decode1_group_kernel<true><<<unsigned(total), NT, lds, s>>>(h);
    else fbi_decode1_group_kernel<false><<<unsigned(total), NT, lds, s>>>(h);
    return hipGetLastError();
}

// The scales of columns j0..j0+3 (j0 a multiple of 4) as two 8-byte words,
// loaded without a branch so that the loads can be issued early: bytes 4 j0
// and 4 j0 + 8 for fp32, byte 2 j0 twice for fp16. alpha is 16-byte aligned,
// so a read past the N-th scale stays inside the aligned 16 bytes holding
// scale j0; j0 >= N reads scale 0.
BGB_DEV void alpha4_load(const void* alpha, int alpha_f16, int64_t j0, int64_t N, uint2 (&raw)[2]) {
    j0 = j0 < N ? j0 : 0;
    const char* a8 = static_cast<const char*>(alpha);
    raw[0] = *reinterpret_cast<const uint2*>(a8 + (alpha_f16 ? 2 * j0 : 4 * j0));
    raw[1] = *reinterpret_cast<const uint2*>(a8 + (alpha_f16 ? 2 * j0 : 4 * j0 + 8));
}
BGB_DEV float alpha4_get(const uint2 (&raw)[2], int alpha_f16, int i) {
    const uint32_t aw[4] = {raw[0].x, raw[0].y, raw[1].x, raw[1].y};
    return alpha_f16 ? f16_to_f32(uint16_t(aw[i >> 1] >> (16 * (i & 1)))) : __uint_as_float(aw[i]);
}

// A few tokens (2 <= M <= 16), activation staging fused: every block copies
// the M tokens into LDS in the decode layout (per token, rows 32t + u and
// 32t + u + 16 side by side), then takes its column group(s) as the
// single-token kernel does. The signs decode to +-1 directly (no per-type
// activation sums): for MFMA u, dword e of the A operand is word e's bit u as
// the sign of the low 16-bit value and bit u + 16 as that of the high one,
// over the bit pattern of 1.0.
constexpr int kDmMaxTokens = 16;
constexpr int kDmWaves = 8;
constexpr int kDmLdsBytes = 140 * 1024;              // staged tokens: [M][Kp + 8] 16-bit values
constexpr int kDmMaxJobs = 2;                        // 256-byte token tiles per thread
constexpr int kDmSeqMinTokens = 8;                   // sequential column groups from this many tokens

// The body is shared by the one-linear kernel (bid, nblk = the block index
// and count) and the grouped one (the block's rank and count within its
// linear). LDS: xs [kDmLdsBytes / 2], xzero [128] (the B operand of steps
// past the last tile), red [2 NW 64] when KQ > 1. kSeq (with IT == 1): a
// block takes seq column groups one after another (bid + q nblk, q < seq) on
// one staging of the tokens; group q + 1's sign tiles and scales are
// requested into a second set of registers while group q runs.
template <bool kF16, bool kTileJobs, int F, int S, int IT, bool kSeq = false>
BGB_DEV void fbi_decodem_body(const uint16_t* __restrict__ x, int M, int64_t K, int64_t N, int64_t TQ,
                              const uint32_t* __restrict__ P, const void* __restrict__ alpha, int alpha_f16,
                              void* __restrict__ y, int y_dtype, int64_t bid, int64_t nblk, uint16_t* xs,
                              uint16_t* xzero, f32x4_t* red, int seq = 1) {
    static_assert(!kSeq || IT == 1, "sequential column groups take one group at a time");
    constexpr int NW = kDmWaves, NT = NW * 64;
    constexpr int KQ = NW / F;
    static_assert(NW % F == 0 && IT * S <= kD1MaxTiles, "few-token W1A16 shape");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r = lane & 15, f = wave % F, kq = wave / F;
    const int64_t ngroups = (N + 16 * F - 1) / (16 * F);
    const int Kp = int(TQ * 128);
    const int stride = Kp + 8;                           // 16 bytes apart: token rows fall in different banks
    const int64_t steps = (TQ + 3) / 4;
    const int Ki = int(K);

    // 1.-2. the tokens into the decode layout (rows 32t + u and 32t + u + 16
    //    side by side, see the single-token kernel). The sign tiles are
    //    requested once the tokens are in. Rows past K read as zeros.
    u32x4_t w[IT][S];
    auto preload_all = [&]() {
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));     // vmcnt(0): the tokens are in
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int64_t grp = bid + int64_t(it) * nblk;
            const int64_t jj = grp < ngroups ? grp * 16 * F + 16 * f + r : N;
            preload<S>(w[it], P, kq, KQ, steps, TQ, N, jj, g);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto load16 = [&](int m, int k, bool ok) {
        ok = ok && k < Ki;
        const u32x4_t t = *reinterpret_cast<const u32x4_t*>(x + (ok ? int64_t(m) * Ki + k : 0));
        return t & u32x4_t(0u - uint32_t(ok));
    };
    if (tid < 16) reinterpret_cast<u32x4_t*>(xzero)[tid] = u32x4_t{0u, 0u, 0u, 0u};
    const int tiles = M * int(TQ);
    if constexpr (kTileJobs) {
        // at least one 128-row tile per thread: job J is tile J / M of token
        // J % M (neighbouring lanes write different tokens' rows, different
        // banks); chunk u of a tile holds, for e = 0..3, rows 32e + u and
        // 32e + u + 16 as one dword, both in dword (u % 8) / 2, same half, of
        // the 16-byte pieces 4e + u / 8 and 4e + 2 + u / 8: one v_perm per
        // dword, 16 16-byte LDS writes per tile
        u32x4_t xv[kDmMaxJobs][16];
#pragma unroll
        for (int i = 0; i < kDmMaxJobs; ++i) {
            if (i * NT >= tiles) break;                  // uniform
            const int J = i * NT + tid, m = J % M, tq = J / M;
#pragma unroll
            for (int j = 0; j < 16; ++j) xv[i][j] = load16(m, 128 * tq + 8 * j, J < tiles);
        }
        preload_all();
#pragma unroll
        for (int i = 0; i < kDmMaxJobs; ++i) {
            if (i * NT >= tiles) break;
            const int J = i * NT + tid;
            if (J >= tiles) continue;
            const int m = J % M, tq = J / M;
            u32x4_t* dst = reinterpret_cast<u32x4_t*>(xs + m * stride + tq * 128);
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int d = (u % 8) / 2;
                const uint32_t sel = (u & 1) ? 0x07060302u : 0x05040100u;
                u32x4_t o;
                o.x = __builtin_amdgcn_perm(xv[i][2 + u / 8][d], xv[i][0 + u / 8][d], sel);
                o.y = __builtin_amdgcn_perm(xv[i][6 + u / 8][d], xv[i][4 + u / 8][d], sel);
                o.z = __builtin_amdgcn_perm(xv[i][10 + u / 8][d], xv[i][8 + u / 8][d], sel);
                o.w = __builtin_amdgcn_perm(xv[i][14 + u / 8][d], xv[i][12 + u / 8][d], sel);
                dst[u] = o;
            }
        }
    } else {
        // fewer tiles than threads: one 16-byte piece (8 rows) per job, piece p
        // of token p / ppt, its 8 values scattered 16 bytes apart
        const int ppt = int(TQ) * 16, pieces = M * ppt;
        u32x4_t xv[kDmMaxJobs * 8];
#pragma unroll
        for (int i = 0; i < kDmMaxJobs * 8; ++i) {
            if (i * NT >= pieces) break;
            const int p = i * NT + tid, m = p / ppt;
            xv[i] = load16(m, 8 * (p - m * ppt), p < pieces);
        }
        preload_all();
#pragma unroll
        for (int i = 0; i < kDmMaxJobs * 8; ++i) {
            if (i * NT >= pieces) break;
            const int p = i * NT + tid;
            if (p >= pieces) continue;
            const int m = p / ppt, k = 8 * (p - m * ppt), t = k >> 5, bq = k & 31;
            uint16_t* dst = xs + m * stride + (t >> 2) * 128 + (bq & 15) * 8 + (t & 3) * 2 + (bq >> 4);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                dst[8 * e] = uint16_t(e & 1 ? xv[i][e >> 1] >> 16 : xv[i][e >> 1] & 0xffffu);
        }
    }
    __syncthreads();

    // 3. per column group: the product for this lane's token r (lanes r >= M
    //    read token 0; their outputs are never stored), the KQ parts' sums
    //    through LDS, the epilogue
    constexpr uint32_t kOne = kF16 ? 0x3C003C00u : 0x3F803F80u;
    const uint16_t* xrow = xs + (r < M ? r : 0) * stride;
    uint2 araw[IT][2];                                  // this lane's 4 column scales per group
#pragma unroll
    for (int it = 0; it < IT; ++it)
        alpha4_load(alpha, alpha_f16, (bid + int64_t(it) * nblk) * 16 * F + 16 * f + 4 * g, N,
                    araw[it]);
    const int nseq = kSeq ? seq : 1;
    u32x4_t wn[kSeq ? S : 1];                           // the next sequential group's tiles
    uint2 arawn[2] = {};
    for (int q = 0; q < nseq; ++q) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int64_t grp = bid + int64_t(it + q) * nblk;   // q > 0 only with kSeq
        if (grp >= ngroups) break;
        if constexpr (kSeq) {
            const int64_t g2 = grp + nblk;
            if (q + 1 < nseq && g2 < ngroups) {
                preload<S>(wn, P, kq, KQ, steps, TQ, N, g2 * 16 * F + 16 * f + r, g);
                alpha4_load(alpha, alpha_f16, g2 * 16 * F + 16 * f + 4 * g, N, arawn);
            }
        }
        const int rb = (it + q) & 1;                      // reduce buffer: alternates between groups
        f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};   // by u parity
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const int64_t st = kq + int64_t(KQ) * i;
            const int64_t tq = st * 4 + g;
            // a step past the column's tiles has zero sign words (all -1): it
            // must read zero activations
            const u32x4_t* src = reinterpret_cast<const u32x4_t*>(st < steps && tq < TQ ? xrow + tq * 128 : xzero);
            const u32x4_t wv = w[it][i];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                u32x4_t a;   // (~(word << (15 - u)) & 0x80008000) | 1.0: signs of rows 32e + u, 32e + u + 16
                a.x = __builtin_amdgcn_bitop3_b32(wv.x << (15 - u), 0x80008000u, kOne, 0xAE);
                a.y = __builtin_amdgcn_bitop3_b32(wv.y << (15 - u), 0x80008000u, kOne, 0xAE);
                a.z = __builtin_amdgcn_bitop3_b32(wv.z << (15 - u), 0x80008000u, kOne, 0xAE);
                a.w = __builtin_amdgcn_bitop3_b32(wv.w << (15 - u), 0x80008000u, kOne, 0xAE);
                acc[u & 1] = mfma16<kF16>(a, src[u], acc[u & 1]);
            }
        }
        f32x4_t z = acc[0] + acc[1];
        if constexpr (KQ > 1) {
            red[(rb * NW + wave) * 64 + lane] = z;
            __syncthreads();
            if (kq != 0 || r >= M) continue;
            // the parts in a fixed order: kq = 0, 1, ..., KQ - 1
#pragma unroll
            for (int kp = 1; kp < KQ; ++kp) z += red[(rb * NW + f + F * kp) * 64 + lane];
        } else {
            if (r >= M) continue;
        }
        const int64_t j0 = grp * 16 * F + 16 * f + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t col = j0 + i;
            if (col >= N) continue;
            store_y(y, y_dtype, int64_t(r) * N + col, alpha4_get(araw[it], alpha_f16, i) * z[i]);
        }
    }
    if constexpr (kSeq) {                               // the prefetched group becomes the current one
        if (q + 1 >= nseq || bid + int64_t(q + 1) * nblk >= ngroups) break;
#pragma unroll
        for (int i = 0; i < S; ++i) w[0][i] = wn[i];
        araw[0][0] = arawn[0];
        araw[0][1] = arawn[1];
    }
    }
}

template <bool kF16, bool kTileJobs, int F, int S, int IT>
__global__ void __launch_bounds__(kDmWaves * 64)
fbi_decodem_kernel(const uint16_t* __restrict__ x, int M, int64_t K, int64_t N, int64_t TQ,
                   const uint32_t* __restrict__ P, const void* __restrict__ alpha, int alpha_f16,
                   void* __restrict__ y, int y_dtype) {
    constexpr int KQ = kDmWaves / F;
    __shared__ __attribute__((aligned(16))) uint16_t xs[kDmLdsBytes / 2];
    __shared__ __attribute__((aligned(16))) uint16_t xzero[128];
    __shared__ f32x4_t red[(KQ > 1 ? 2 * kDmWaves : 1) * 64];
    fbi_decodem_body<kF16, kTileJobs, F, S, IT>(x, M, K, N, TQ, P, alpha, alpha_f16, y, y_dtype, blockIdx.x,
                                                gridDim.x, xs, xzero, red);
}

bool w1a16_decodem_supported(int64_t M, int64_t K) {
    if (M < 2 || M > kDmMaxTokens) return false;
    const int64_t Kp = padded_k(K);
    // the tokens fit in LDS; at most 2 tiles per thread to stage; and at most
    // kD1MaxTiles steps per wave when the 8 waves share one fragment's K range
    return M * (Kp + 8) * 2 <= kDmLdsBytes && M * (Kp / 128) <= int64_t(kDmMaxJobs) * kDmWaves * 64 &&
           Kp <= int64_t(kD1MaxTiles) * kDmWaves * 4 * 128;
}

template <bool kF16, bool kTJ, int F, int S>
static void launch_w1a16_decodem_s(int it, unsigned grid, const uint16_t* x, int M, int64_t K, int64_t N,
                                   int64_t TQ, const uint32_t* P, const void* alpha, int alpha_f16, void* y,
                                   int y_dtype, hipStream_t s) {
#define BGB_DMX(ITV)                                                                                           \
    fbi_decodem_kernel<kF16, kTJ, F, S, ITV><<<grid, kDmWaves * 64, 0, s>>>(x, M, K, N, TQ, P, alpha, alpha_f16, y, \
                                                                        y_dtype)
    if constexpr (2 * S <= kD1MaxTiles) {
        if (it == 2) {
            BGB_DMX(2);
            return;
        }
    }
    BGB_DMX(1);
#undef BGB_DMX
}

template <bool kF16, bool kTJ, int F>
static void launch_w1a16_decodem_f(int S, int it, unsigned grid, const uint16_t* x, int M, int64_t K, int64_t N,
                                   int64_t TQ, const uint32_t* P, const void* alpha, int alpha_f16, void* y,
                                   int y_dtype, hipStream_t s) {
#define BGB_DMS(SV) launch_w1a16_decodem_s<kF16, kTJ, F, SV>(it, grid, x, M, K, N, TQ, P, alpha, alpha_f16, y, y_dtype, s)
    if (S == 1) BGB_DMS(1);
    else if (S == 2) BGB_DMS(2);
    else if (S == 4) BGB_DMS(4);
    else BGB_DMS(8);
#undef BGB_DMS
}

template <bool kF16, bool kTJ>
static hipError_t launch_w1a16_decodem_t(const uint16_t* x, int M, int64_t K, int64_t N, const uint32_t* P,
                                         const void* alpha, int alpha_f16, void* y, int y_dtype, hipStream_t s) {
    const int64_t TQ = tiles_per_col(K);
    const int64_t steps = (TQ + 3) / 4;
    const int64_t frags = (N + 15) / 16;
    // steps per wave for F fragments per group: the NW / F waves of a
    // fragment share the steps (a power of two, at most 8 tiles per thread)
    auto steps_per_wave = [&](int f) {
        const int64_t need = (steps + kDmWaves / f - 1) / (kDmWaves / f);
        return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 16;
    };
    // the fewest fragments per group that give each block one group; else
    // the most allowed and up to two groups per block
    int F = 1;
    while (2 * F <= kDmWaves && steps_per_wave(2 * F) <= kD1MaxTiles && (frags + F - 1) / F > kD1MaxGrid) F *= 2;
    const int S = steps_per_wave(F);
    if (S > kD1MaxTiles) return hipErrorInvalidValue;   // K beyond the fused size (not reached: supported())
    const int64_t groups = (frags + F - 1) / F;
    int64_t grid = groups < kD1MaxGrid ? groups : kD1MaxGrid;
    int it = int((groups + grid - 1) / grid);
    const int it_max = 2 * S <= kD1MaxTiles ? 2 : 1;
    if (it > it_max) {
        it = it_max;
        grid = (groups + it - 1) / it;
    }
    const unsigned gr = unsigned(grid);
#define BGB_DMF(FV) launch_w1a16_decodem_f<kF16, kTJ, FV>(S, it, gr, x, M, K, N, TQ, P, alpha, alpha_f16, y, y_dtype, s)
    if (F == 1) BGB_DMF(1);
    else if (F == 2) BGB_DMF(2);
    else if (F == 4) BGB_DMF(4);
    else BGB_DMF(8);
#undef BGB_DMF
    return hipGetLastError();
}

hipError_t launch_w1a16_decodem(const void* x, int x_f16, int64_t M, int64_t K, int64_t N, const uint32_t* P,
                                const void* alpha, int alpha_f16, void* y, int y_dtype, hipStream_t s) {
    if (!w1a16_decodem_supported(M, K)) return hipErrorInvalidValue;
    const uint16_t* xx = static_cast<const uint16_t*>(x);
    // whole tiles per thread once there is at least one per thread
    const bool tj = M * tiles_per_col(K) >= kDmWaves * 64;
    const int m = int(M);
    if (x_f16) return tj ? launch_w1a16_decodem_t<true, true>(xx, m, K, N, P, alpha, alpha_f16, y, y_dtype, s)
                         : launch_w1a16_decodem_t<true, false>(xx, m, K, N, P, alpha, alpha_f16, y, y_dtype, s);
    return tj ? launch_w1a16_decodem_t<false, true>(xx, m, K, N, P, alpha, alpha_f16, y, y_dtype, s)
              : launch_w1a16_decodem_t<false, false>(xx, m, K, N, P, alpha, alpha_f16, y, y_dtype, s);
}

// Several independent linears of 2..16 tokens in one launch: each linear
// keeps the split of its own launch (F fragments per group, S steps per
// wave, one group per block), the grid is the concatenation of the linears'
// blocks (most sign bytes per block first), and a block finds its linear by
// uniform selects over the table in the kernel arguments. Each item keeps its
// own staging form too (16-byte pieces, or whole 128-row tiles once there
// are as many tiles as threads).
struct DmItem {
    const uint16_t* x;
    const uint32_t* P;
    const void* alpha;
    void* y;
    int64_t K, N, TQ;
    int first, nblk, cfg;   // first block, block count, (staging, F, S) case
    int seq;                // column groups per block, one after another
};
struct DmGroup {
    DmItem it[kGroupMax];
    int count, M, alpha_f16, y_dtype;
};

template <bool kF16>
__global__ void __launch_bounds__(kDmWaves * 64)
fbi_decodem_group_kernel(const DmGroup g) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[kDmLdsBytes / 2];
    __shared__ __attribute__((aligned(16))) uint16_t xzero[128];
    __shared__ f32x4_t red[2 * kDmWaves * 64];
    DmItem it = g.it[0];
#pragma unroll
    for (int i = 1; i < kGroupMax; ++i)
        if (i < g.count && int(blockIdx.x) >= g.it[i].first) it = g.it[i];
    const int64_t bid = int64_t(blockIdx.x) - it.first;
#define BGB_GM(C, TJ, FV, SV)                                                                                     \
    case C:                                                                                                    \
        fbi_decodem_body<kF16, TJ, FV, SV, 1>(it.x, g.M, it.K, it.N, it.TQ, it.P, it.alpha, g.alpha_f16, it.y,   \
                                              g.y_dtype, bid, it.nblk, xs, xzero, red);                        \
        break;                                                                                                 \
    case 32 + C:                                                                                               \
        fbi_decodem_body<kF16, TJ, FV, SV, 1, true>(it.x, g.M, it.K, it.N, it.TQ, it.P, it.alpha, g.alpha_f16,   \
                                                    it.y, g.y_dtype, bid, it.nblk, xs, xzero, red, it.seq);    \
        break;
    switch (it.cfg) {
        BGB_GM(0, false, 1, 1) BGB_GM(1, false, 1, 2) BGB_GM(2, false, 1, 4) BGB_GM(3, false, 1, 8)
        BGB_GM(4, false, 2, 1) BGB_GM(5, false, 2, 2) BGB_GM(6, false, 2, 4) BGB_GM(7, false, 2, 8)
        BGB_GM(8, false, 4, 1) BGB_GM(9, false, 4, 2) BGB_GM(10, false, 4, 4) BGB_GM(11, false, 4, 8)
        BGB_GM(12, false, 8, 1) BGB_GM(13, false, 8, 2) BGB_GM(14, false, 8, 4) BGB_GM(15, false, 8, 8)
        BGB_GM(16, true, 1, 1) BGB_GM(17, true, 1, 2) BGB_GM(18, true, 1, 4) BGB_GM(19, true, 1, 8)
        BGB_GM(20, true, 2, 1) BGB_GM(21, true, 2, 2) BGB_GM(22, true, 2, 4) BGB_GM(23, true, 2, 8)
        BGB_GM(24, true, 4, 1) BGB_GM(25, true, 4, 2) BGB_GM(26, true, 4, 4) BGB_GM(27, true, 4, 8)
        BGB_GM(28, true, 8, 1) BGB_GM(29, true, 8, 2) BGB_GM(30, true, 8, 4) BGB_GM(31, true, 8, 8)
        default: break;
    }
#undef BGB_GM
}

bool w1a16_decodem_group_supported(const W1a16Item* items, int count, int64_t M) {
    if (count < 0 || count > kGroupMax) return false;
    for (int i = 0; i < count; ++i) {
        if (items[i].N <= 0) continue;
        if (!w1a16_decodem_supported(M, items[i].K)) return false;
    }
    return true;
}

hipError_t launch_w1a16_decodem_group(const W1a16Item* items, int count, int64_t M, int x_f16, int alpha_f16,
                                      int y_dtype, hipStream_t s) {
    if (!w1a16_decodem_group_supported(items, count, M)) return hipErrorInvalidValue;
    DmGroup g{};
    int order[kGroupMax], n = 0;
    int Fs[kGroupMax];
    int64_t cost[kGroupMax], frag[kGroupMax], stp[kGroupMax];
    auto spw = [&](int i, int f) {                           // steps per wave, as the one-linear launcher
        const int64_t need = (stp[i] + kDmWaves / f - 1) / (kDmWaves / f);
        return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 16;
    };
    auto grows = [&](int i) { return 2 * Fs[i] <= kDmWaves && spw(i, 2 * Fs[i]) <= kD1MaxTiles; };
    int64_t total_blocks = 0;
    for (int i = 0; i < count; ++i) {
        if (items[i].N <= 0) continue;
        const W1a16Item& in = items[i];
        DmItem& d = g.it[n];
        d.x = static_cast<const uint16_t*>(in.x);
        d.P = in.P;
        d.alpha = in.alpha;
        d.y = in.y;
        d.K = in.K;
        d.N = in.N;
        d.TQ = tiles_per_col(in.K);
        stp[n] = (d.TQ + 3) / 4;
        frag[n] = (in.N + 15) / 16;
        Fs[n] = 1;                                           // enough blocks for the linear alone to fill the chip
        while (grows(n) && (frag[n] + Fs[n] - 1) / Fs[n] > kD1MaxGrid) Fs[n] *= 2;
        total_blocks += (frag[n] + Fs[n] - 1) / Fs[n];
        order[n] = n;
        ++n;
    }
    // Every block stages all the tokens before any product and a block fills
    // a CU's LDS, so a grid beyond one block per CU repeats that staging in
    // later rounds: widen the groups of the linear with the most blocks until
    // the grid fits or none can widen.
    while (total_blocks > kD1MaxGrid) {
        int best = -1;
        for (int i = 0; i < n; ++i)
            if (grows(i) && (best < 0 || (frag[i] + Fs[i] - 1) / Fs[i] > (frag[best] + Fs[best] - 1) / Fs[best]))
                best = i;
        if (best < 0) break;
        total_blocks -= (frag[best] + Fs[best] - 1) / Fs[best];
        Fs[best] *= 2;
        total_blocks += (frag[best] + Fs[best] - 1) / Fs[best];
    }
    // Still more blocks than CUs (every item at its widest groups): rather
    // than a second round that stages the tokens again, blocks take several
    // column groups one after another. The smallest cap C on a block's work
    // (fragments x 128-row tiles) whose plan fits one block per CU: per item
    // the fragments per group F (its widest groups or half as wide, so that
    // a group's barrier and reduction stay few) and seq = C / (F TQ) groups
    // per block, whichever F gives the fewest blocks. More work per block
    // means fewer blocks, so C is found by bisection. Only from 8 tokens:
    // below that the staging is cheap (4 tokens of 4096: 32 KB per block) and
    // the groups' extra barriers and reductions cost more than a second round
    // (7B-shaped layer at 4 tokens: 27.7 us with sequential groups against
    // 23.3 us in two rounds; at 16 tokens 36.9 against 43.9 us).
    int seqs[kGroupMax];
    for (int i = 0; i < n; ++i) seqs[i] = 1;
    if (total_blocks > kD1MaxGrid && M >= kDmSeqMinTokens) {
        int fc[kGroupMax], sc[kGroupMax];
        auto fit = [&](int64_t C) {
            int64_t tot = 0;
            for (int i = 0; i < n; ++i) {
                const int64_t tq = g.it[i].TQ;
                int64_t bestb = -1;
                fc[i] = Fs[i];
                sc[i] = 1;
                for (int F = Fs[i] > 1 ? Fs[i] / 2 : 1; F <= Fs[i]; F *= 2) {
                    const int64_t sq = C / (F * tq);
                    if (sq < 1) continue;
                    const int64_t nb = ((frag[i] + F - 1) / F + sq - 1) / sq;
                    if (bestb < 0 || nb <= bestb) {
                        bestb = nb;
                        fc[i] = F;
                        sc[i] = int(sq < (int64_t(1) << 20) ? sq : (int64_t(1) << 20));
                    }
                }
                tot += bestb < 0 ? (frag[i] + Fs[i] - 1) / Fs[i] : bestb;
            }
            return tot <= kD1MaxGrid;
        };
        int64_t lo = 1, hi = 1;
        for (int i = 0; i < n; ++i) hi += int64_t(Fs[i]) * g.it[i].TQ * ((frag[i] + Fs[i] - 1) / Fs[i]);
        while (lo < hi) {                                // smallest C that fits (fit(hi) holds: one block per item)
            const int64_t mid = lo + (hi - lo) / 2;
            if (fit(mid)) hi = mid;
            else lo = mid + 1;
        }
        fit(lo);
        for (int i = 0; i < n; ++i) {
            Fs[i] = fc[i];
            seqs[i] = sc[i];
        }
    }
    for (int i = 0; i < n; ++i) {
        DmItem& d = g.it[i];
        const int F = Fs[i], S = spw(i, F);
        if (S > kD1MaxTiles) return hipErrorInvalidValue;  // not reached: supported()
        d.seq = seqs[i];
        d.nblk = int(((frag[i] + F - 1) / F + seqs[i] - 1) / seqs[i]);
        const bool tj = M * d.TQ >= kDmWaves * 64;          // whole tiles per thread, as the one-linear launcher
        d.cfg = 32 * (seqs[i] > 1) + 16 * tj + 4 * (F == 1 ? 0 : F == 2 ? 1 : F == 4 ? 2 : 3) +
                (S == 1 ? 0 : S == 2 ? 1 : S == 4 ? 2 : 3);
        cost[i] = int64_t(F) * seqs[i] * d.TQ;
    }
    if (n == 0) return hipSuccess;
    for (int a = 1; a < n; ++a)
        for (int b = a; b > 0 && cost[order[b]] > cost[order[b - 1]]; --b) {
            const int t = order[b];
            order[b] = order[b - 1];
            order[b - 1] = t;
        }
    DmGroup h{};
    int64_t total = 0;
    for (int i = 0; i < n; ++i) {
        h.it[i] = g.it[order[i]];
        h.it[i].first = int(total);
        total += h.it[i].nblk;
    }
    h.count = n;
    h.M = int(M);
    h.alpha_f16 = alpha_f16;
    h.y_dtype = y_dtype;
    if (x_f16) fbi_decodem_group_kernel<true><<<unsigned(total), kDmWaves * 64, 0, s>>>(h);
    else fbi_decodem_group_kernel<false><<<unsigned(total), kDmWaves * 64, 0, s>>>(h);
    return hipGetLastError();
}

// Up to 64 tokens, activation staging fused, K in chunks. A block of 8 waves
// takes FB 16-column fragments and up to 32 tokens (TF fragments of 16); K
// goes in chunks of 8 TPW tiles of 128 rows, staged through LDS in the decode
// layout, and wave w takes tiles w, w + 8, ... of each chunk for all FB
// fragments, so an activation operand read from LDS feeds FB MFMAs. Here a
// tile is one MFMA step of its own: lane group g of MFMA v takes bit pair
// (u, u + 16), u = 4v + g, of the tile's 4 words (+-1 over the bit pattern of
// 1.0) and the matching activations, chunk u of the tile. The next chunk's
// activations and sign tiles load while the matrix cores work on this one;
// the 8 waves' partial sums meet in LDS in a fixed order.
constexpr int kDkWaves = 8;
constexpr int kDkChunkElems = 32768;                // tokens x rows staged per chunk

template <bool kF16, int TF, int FB, int TPW>
__global__ void __launch_bounds__(kDkWaves * 64)
fbi_decodek_kernel(const uint16_t* __restrict__ x, int M, int64_t K, int64_t N, int64_t TQ,
                   const uint32_t* __restrict__ P, const void* __restrict__ alpha, int alpha_f16,
                   void* __restrict__ y, int y_dtype, int cps, float* __restrict__ part) {
    constexpr int NW = kDkWaves, NT = NW * 64;
    constexpr int MB = 16 * TF;                         // tokens per block
    constexpr int CT = NW * TPW;                        // tiles per chunk
    constexpr int Kc = 128 * CT;                        // rows per chunk
    constexpr int stride = Kc + 16;                     // per token: 32 bytes apart modulo the banks
    constexpr int words = MB * (Kc / 32);               // staging jobs per chunk: 32-row words
    static_assert(MB * Kc <= kDkChunkElems && words <= 2 * NT, "chunk size");   // jobs per thread <= 2
    __shared__ __attribute__((aligned(16))) uint16_t xs[MB * stride];
    __shared__ f32x4_t red[NW][FB * TF][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int m0 = int(blockIdx.y) * MB;                // first token of this block
    const int mb = M - m0 < MB ? M - m0 : MB;           // its tokens
    const int64_t j0 = int64_t(blockIdx.x) * 16 * FB;   // first column
    const int Ki = int(K);
    const int nchunks = int((TQ + CT - 1) / CT);
    // this block's chunks: split z = blockIdx.z takes [c0, c1)
    const int c0 = int(blockIdx.z) * cps;
    const int c1 = c0 + cps < nchunks ? c0 + cps : nchunks;

    // chunk c's rows of the block's tokens (rows past K are zeroed when
    // stored) and this wave's sign
    // tiles of it (tile c CT + w + 8p, column j0 + 16f + r; past TQ or N they
    // read tile 0 of column 0: their activations are zero, their outputs are
    // never stored)
    // Job J is the 32-row word t of token m with m % 4 = J % 4 and
    // t % 4 = (J / 4) % 4, so that the 16-lane groups of a store write 16
    // different banks (the token stride is 8 dwords modulo 32).
    const int mq = (mb + 3) / 4;                        // token quads
    auto job = [&](int J, int& m, int& t) {
        const int rest = J >> 4;
        m = 4 * (rest % mq) + (J & 3);
        t = 4 * (rest / mq) + ((J >> 2) & 3);
        return m < mb && t < Kc / 32;
    };
    u32x4_t xv[2][4], wn[TPW][FB];
    auto load_chunk = [&](int c) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int m, t;
            const bool jv = job(i * NT + tid, m, t);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = c * Kc + 32 * t + 8 * j;
                const bool ok = jv && k < Ki;
                xv[i][j] = *reinterpret_cast<const u32x4_t*>(x + (ok ? int64_t(m0 + m) * Ki + k : 0));
            }
        }
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
            const int64_t tq = int64_t(c) * CT + wave + NW * p;
#pragma unroll
            for (int f = 0; f < FB; ++f) {
                const int64_t j = j0 + 16 * f + r;
                const bool ok = tq < TQ && j < N;
                wn[p][f] = load_tile(P, ok ? tq : 0, N, ok ? j : 0);
            }
        }
    };
    auto store_chunk = [&](int c) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int m, t;
            if (!job(i * NT + tid, m, t)) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (c * Kc + 32 * t + 8 * j >= Ki) xv[i][j] = u32x4_t{0u, 0u, 0u, 0u};
            // dword u of the tile's chunk u (here: 16 bytes apart) holds rows u, u + 16
            // of the word: dword (u % 8) / 2, same half, of pieces u / 8 and 2 + u / 8
            uint32_t* dst = reinterpret_cast<uint32_t*>(xs + m * stride + (t >> 2) * 128 + (t & 3) * 2);
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const uint32_t sel = (u & 1) ? 0x07060302u : 0x05040100u;
                dst[4 * u] = __builtin_amdgcn_perm(xv[i][2 + u / 8][(u % 8) / 2], xv[i][u / 8][(u % 8) / 2], sel);
            }
        }
    };
    load_chunk(c0);
    // the reducing wave's 4 column scales (wave q < FB TF finishes fragment q / TF)
    uint2 araw[2];
    alpha4_load(alpha, alpha_f16, j0 + 16 * (wave / TF) + 4 * g, N, araw);

    constexpr uint32_t kOne = kF16 ? 0x3C003C00u : 0x3F803F80u;
    f32x4_t acc[FB][TF][2];                             // by MFMA parity: two chains each
#pragma unroll
    for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int tf = 0; tf < TF; ++tf) acc[f][tf][0] = acc[f][tf][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const uint16_t* xrow[TF];                           // lanes past the block's tokens read its token 0
#pragma unroll
    for (int tf = 0; tf < TF; ++tf) xrow[tf] = xs + (16 * tf + r < mb ? 16 * tf + r : 0) * stride;

    for (int c = c0; c < c1; ++c) {
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));     // vmcnt(0): chunk c is in
        store_chunk(c);
        u32x4_t w[TPW][FB];
#pragma unroll
        for (int p = 0; p < TPW; ++p)
#pragma unroll
            for (int f = 0; f < FB; ++f) w[p][f] = wn[p][f];
        __syncthreads();
        if (c + 1 < c1) load_chunk(c + 1);
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
            const int tl = wave + NW * p;                  // tile within the chunk (zero rows past K)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int u = 4 * v + g;
                u32x4_t b[TF];
#pragma unroll
                for (int tf = 0; tf < TF; ++tf) b[tf] = *reinterpret_cast<const u32x4_t*>(xrow[tf] + tl * 128 + u * 8);
#pragma unroll
                for (int f = 0; f < FB; ++f) {
                    u32x4_t a;   // (~(word << (15 - u)) & 0x80008000) | 1.0: signs of rows 32e + u, 32e + u + 16
                    a.x = __builtin_amdgcn_bitop3_b32(w[p][f].x << (15 - u), 0x80008000u, kOne, 0xAE);
                    a.y = __builtin_amdgcn_bitop3_b32(w[p][f].y << (15 - u), 0x80008000u, kOne, 0xAE);
                    a.z = __builtin_amdgcn_bitop3_b32(w[p][f].z << (15 - u), 0x80008000u, kOne, 0xAE);
                    a.w = __builtin_amdgcn_bitop3_b32(w[p][f].w << (15 - u), 0x80008000u, kOne, 0xAE);
#pragma unroll
                    for (int tf = 0; tf < TF; ++tf)
                        acc[f][tf][v & 1] = mfma16<kF16>(a, b[tf], acc[f][tf][v & 1]);
                }
            }
        }
        __syncthreads();                                // chunk c's buffer is free again
    }

    // the 8 waves' sums in wave order, by wave q < FB TF for (fragment q / TF,
    // token fragment q % TF), then the epilogue
#pragma unroll
    for (int f = 0; f < FB; ++f)
#pragma unroll
        for (int tf = 0; tf < TF; ++tf) red[wave][f * TF + tf][lane] = acc[f][tf][0] + acc[f][tf][1];
    __syncthreads();
    if (wave >= FB * TF) return;
    const int f = wave / TF, tf = wave % TF;
    f32x4_t z = red[0][wave][lane];
#pragma unroll
    for (int q = 1; q < NW; ++q) z += red[q][wave][lane];
    const int m = 16 * tf + r;
    if (m >= mb) return;
    if (part) {                                         // raw sums of split z, [z][M][N]
        float* dst = part + (int64_t(blockIdx.z) * M + m0 + m) * N;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t col = j0 + 16 * f + 4 * g + i;
            if (col < N) dst[col] = z[i];
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t col = j0 + 16 * f + 4 * g + i;
        if (col >= N) continue;
        store_y(y, y_dtype, int64_t(m0 + m) * N + col, alpha4_get(araw, alpha_f16, i) * z[i]);
    }
}

constexpr int kDkMaxTokens = 64;

bool w1a16_decodek_supported(int64_t M, int64_t K) { return M >= 1 && M <= kDkMaxTokens && K > 0; }

// Launch plan. Measured on the chunked kernel: about 3.6 us of fixed cost
// (launch, first loads, epilogue) plus about 2.4 us per chunk of 32768 staged
// elements (32 tokens x 1024 rows; a chunk of 16 tokens x 1024 rows costs
// half), at up to one block per CU; a split adds the reduce pass (a launch
// plus its traffic). Splits are chosen to cut the chunks per block while the
// grid stays within one block per CU; more fragments per block (each
// activation read feeding more MFMAs) are preferred at equal cost. Chunks are
// one tile per wave: at 16 tokens, two tiles per wave (2048-row chunks) left
// the 16-token 11008 x 4096 linear at 3 splits of 2 chunks on 192 blocks,
// 1.5 us slower than 4 splits of 3 chunks on 256.
namespace {
constexpr double kDkFixedUs = 3.6, kDkChunkUs = 2.4, kDkReduceUs = 2.5, kDkReduceBytesPerUs = 4.0e6;
constexpr int kDkMaxBlocks = 256;
}  // namespace

DecodekPlan decodek_plan(int64_t M, int64_t K, int64_t N) {
    DecodekPlan p{};
    p.tf = M <= 16 ? 1 : 2;                  // 16 or 32 tokens per block, chunks of 8 tiles
    p.tpw = 1;
    const int64_t TQ = tiles_per_col(K);
    const int CT = kDkWaves * p.tpw;
    p.nchunks = int((TQ + CT - 1) / CT);
    const double chunk_us = kDkChunkUs * double(16 * p.tf * 128 * CT) / double(kDkChunkElems);
    const int64_t frags = (N + 15) / 16;
    const int64_t tblocks = (M + 16 * p.tf - 1) / (16 * p.tf);
    double best = 1e300;
    for (int fb : {4, 2, 1}) {
        const int64_t cb = (frags + fb - 1) / fb;
        for (int S = 1; S <= p.nchunks; ++S) {
            const int cps = (p.nchunks + S - 1) / S;
            const int splits = (p.nchunks + cps - 1) / cps;
            if (splits != S) continue;                       // same split count as a smaller S
            const int64_t blocks = cb * tblocks * splits;
            const double rounds = double((blocks + kDkMaxBlocks - 1) / kDkMaxBlocks);
            double t = kDkFixedUs + rounds * cps * chunk_us;
            if (splits > 1) t += kDkReduceUs + double(splits + 1) * double(M) * double(N) * 4.0 / kDkReduceBytesPerUs;
            if (blocks < 128 && fb > 1) t += blocks < 64 ? 1.0 : 0.3;   // few CUs streaming the signs
            if (t < best - 1e-9) {
                best = t;
                p.fb = fb;
                p.splits = splits;
                p.cps = cps;
            }
        }
    }
    return p;
}

size_t w1a16_decode_ws_bytes(int64_t M, int64_t K, int64_t N) {
    if (M < 1 || M > kW1A16DecodeMaxM || N < 1) return 0;
    if ((M == 1 && w1a16_decode1_supported(K)) || w1a16_decodem_supported(M, K)) return 0;
    const DecodekPlan p = decodek_plan(M, K, N);
    return p.splits > 1 ? align256(size_t(p.splits) * size_t(M) * size_t(N) * 4) : 0;
}

template <bool kF16, int TF, int TPW>
static hipError_t launch_w1a16_decodek_t(const DecodekPlan& p, const uint16_t* x, int M, int64_t K, int64_t N,
                                         const uint32_t* P, const void* alpha, int alpha_f16, void* y, int y_dtype,
                                         float* part, hipStream_t s) {
    constexpr int MB = 16 * TF;
    const int64_t TQ = tiles_per_col(K);
    const int64_t frags = (N + 15) / 16;
    const int tblocks = (M + MB - 1) / MB;
    const dim3 grid = dim3(unsigned((frags + p.fb - 1) / p.fb), unsigned(tblocks), unsigned(p.splits));
    float* pt = p.splits > 1 ? part : nullptr;
#define BGB_DK(FBV)                                                                                              \
    fbi_decodek_kernel<kF16, TF, FBV, TPW><<<grid, kDkWaves * 64, 0, s>>>(x, M, K, N, TQ, P, alpha, alpha_f16, y, \
                                                                           y_dtype, p.cps, pt)
    if (p.fb == 4) BGB_DK(4);
    else if (p.fb == 2) BGB_DK(2);
    else BGB_DK(1);
#undef BGB_DK
    if (p.splits > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_w1a16_splitk_reduce(part, p.splits, M, N, alpha, alpha_f16, y, y_dtype, s);
    }
    return hipGetLastError();
}

hipError_t launch_w1a16_decodek(const void* x, int x_f16, int64_t M, int64_t K, int64_t N, const uint32_t* P,
                                const void* alpha, int alpha_f16, void* y, int y_dtype, float* part,
                                hipStream_t s) {
    if (!w1a16_decodek_supported(M, K)) return hipErrorInvalidValue;
    const DecodekPlan p = decodek_plan(M, K, N);
    if (p.splits > 1 && !part) return hipErrorInvalidValue;
    const uint16_t* xx = static_cast<const uint16_t*>(x);
    const int m = int(M);
    if (p.tf == 1)
        return x_f16 ? launch_w1a16_decodek_t<true, 1, 1>(p, xx, m, K, N, P, alpha, alpha_f16, y, y_dtype, part, s)
                     : launch_w1a16_decodek_t<false, 1, 1>(p, xx, m, K, N, P, alpha, alpha_f16, y, y_dtype, part, s);
    return x_f16 ? launch_w1a16_decodek_t<true, 2, 1>(p, xx, m, K, N, P, alpha, alpha_f16, y, y_dtype, part, s)
                 : launch_w1a16_decodek_t<false, 2, 1>(p, xx, m, K, N, P, alpha, alpha_f16, y, y_dtype, part, s);
}

}  // namespace bgb
