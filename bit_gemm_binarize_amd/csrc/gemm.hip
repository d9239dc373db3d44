// Prefill kernels (M > 64): a dense contraction, so it runs on the matrix
// cores. FBI-linear W1A16 (FBI-LLM news rewrite, FBI-linear paragraph) on
// bf16/f16 MFMA with fp32 accumulation; BitLinear W1A8 ("BitNet b1.58: 1bit
// LLM时代", section 一, eq. (7)) on int8 MFMA with int32 accumulation.
//
// Tiling: a block of 4 waves computes a 256-column x 128-token tile; wave w
// owns columns 64w..64w+63 (four 16-column MFMA fragments) for all 128
// tokens (eight 16-token fragments): 32 accumulators of 16x16.
//
// Pipeline: the K loop runs over stages of 128 bytes of activations per token
// (64 rows of bf16/f16, 128 rows of int8). Activation stages go from global
// memory straight into LDS with global_load_lds_dwordx4 (no VGPR staging),
// four stages in flight in a ring of four 16 KB buffers; the block's 4 KB sign
// tile of a stage goes the same way into a second ring. One s_waitcnt +
// s_barrier per stage; the waits are explicit because only the kernel knows
// how many DMA operations a stage issues.
//
// LDS layout of a stage: token row t at t*128 bytes, its eight 16-byte chunks
// XOR-swizzled by a function of t so that the B-operand reads (a half-wave of
// 32 lanes = 16 token rows x 2 chunks per pass on gfx950's 128-bank LDS) hit
// 32 distinct bank groups. The DMA writes lane L of an instruction to chunk
// base+L, so the swizzle is applied by choosing the source chunk per lane.
//
// Sign decoding (A operand, rows = output columns), per MFMA:
// * W1A16: lane group g takes word g>>1 of the stage and the rows 4u+e and
//   4u+e+16 (u = 2v + (g&1)) as dword e of its operand: one bitop3 of the
//   shifted word gives the two sign bits over the bit pattern of 1.0. The
//   activations were interleaved to match by the prep kernel: within each
//   32-row group, element pair i holds rows i and i+16.
// * W1A8: lane group g takes word g, MFMA v = 0..1, dword d carries rows
//   4v+d+8e (byte e) as 0/1 bytes; sum s q = 2 sum b q - sum q with the row
//   sums of the codes from the prologue, which writes the codes in this order.
#include "bgb_device.hpp"
#include "bgb_internal.hpp"

#include <type_traits>

namespace bgb {

constexpr int kBM = 128;            // tokens per block tile
constexpr int kBJ = 256;            // output columns per block tile
constexpr int kStageBytes = 16384;  // kBM rows x 128 bytes
constexpr int kRing = 4;            // stages in the LDS rings
constexpr int kWTileBytes = kBJ * 16;   // one 128-row sign tile of the block's columns

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

// Chunk swizzles of a stage row (see the header comment); both are
// involutions on 0..7 and depend only on bits 2..3 of the token row.
BGB_DEV int swz16(int t) { return 2 * ((t >> 2) & 3); }
BGB_DEV int swz8(int t) { return ((t >> 2) & 1) | (((t >> 3) & 1) << 2); }

// Per-thread DMA plan: instruction i of wave w moves stage chunks
// (4i+w)*64 .. +63; lane L takes chunk p = (4i+w)*64 + L -> token row p>>3,
// LDS slot p&7, source chunk (p&7) ^ swz(row). Rows past M read row M-1
// (their outputs are never stored).
template <bool k16>
BGB_DEV void dma_plan(const uint8_t* base, int64_t row_bytes, int64_t m0, int64_t M, int tid,
                      const uint8_t* (&src)[4]) {
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = (4 * i + wave) * 64 + lane;
        const int t = p >> 3, slot = p & 7;
        const int c = slot ^ (k16 ? swz16(t) : swz8(t));
        const int64_t m = m0 + t < M ? m0 + t : M - 1;
        src[i] = base + m * row_bytes + 16 * c;
    }
}

BGB_DEV void dma_stage(const uint8_t* const (&src)[4], int64_t off, uint8_t* buf, int wave) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(src[i] + off, buf + (4 * i + wave) * 1024);
}

// Sign tile tq of the block's 256 columns: 16 bytes per column, thread tid
// moves column j0 + tid (clamped to N-1) to byte 16*tid of the LDS tile.
BGB_DEV const uint8_t* wtile_src(const uint32_t* P, int64_t j0, int64_t N, int tid) {
    const int64_t j = j0 + tid < N ? j0 + tid : N - 1;
    return reinterpret_cast<const uint8_t*>(P + j * 4);
}

// ------------------------------------------------------------ W1A16 prep ----
// xi[m][Kp]: within each 32-row group, element 2i = x[m][32t+i] and element
// 2i+1 = x[m][32t+i+16]; rows >= K are zero. One thread per (m, group).
__global__ void __launch_bounds__(256)
w1a16_interleave_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t Kp,
                        uint16_t* __restrict__ xi) {
    const int64_t groups = Kp / 32;
    const int64_t id = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (id >= M * groups) return;
    const int64_t m = id / groups, t = id % groups, k0 = 32 * t;
    const uint16_t* row = x + m * K;
    u32x4_t o[4];
    if ((K & 7) == 0 && k0 + 32 <= K) {
        const u32x4_t* s = reinterpret_cast<const u32x4_t*>(row + k0);
        const u32x4_t l0 = s[0], l1 = s[1], h0 = s[2], h1 = s[3];
        const uint32_t lo[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        const uint32_t hi[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            o[q].x = __builtin_amdgcn_perm(hi[2 * q], lo[2 * q], 0x05040100u);
            o[q].y = __builtin_amdgcn_perm(hi[2 * q], lo[2 * q], 0x07060302u);
            o[q].z = __builtin_amdgcn_perm(hi[2 * q + 1], lo[2 * q + 1], 0x05040100u);
            o[q].w = __builtin_amdgcn_perm(hi[2 * q + 1], lo[2 * q + 1], 0x07060302u);
        }
    } else {
        uint32_t d[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t a = k0 + i < K ? row[k0 + i] : 0u;
            const uint32_t b = k0 + i + 16 < K ? row[k0 + i + 16] : 0u;
            d[i] = a | (b << 16);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = u32x4_t{d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]};
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(xi + m * Kp + k0);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = o[q];
}

hipError_t launch_w1a16_interleave(const void* x, int64_t M, int64_t K, uint16_t* xi, hipStream_t s) {
    const int64_t Kp = padded_k(K), n = M * (Kp / 32);
    w1a16_interleave_kernel<<<unsigned((n + 255) / 256), 256, 0, s>>>(static_cast<const uint16_t*>(x), M, K, Kp, xi);
    return hipGetLastError();
}

// ------------------------------------------------------------------ W1A16 ----
BGB_DEV float alpha_at(const void* alpha, int alpha_f16, int64_t j) {
    return alpha_f16 ? f16_to_f32(static_cast<const uint16_t*>(alpha)[j]) : static_cast<const float*>(alpha)[j];
}

template <bool kF16>
__global__ void __launch_bounds__(256, 2)
gemm_w1a16_kernel(const uint16_t* __restrict__ xi, int64_t M, int64_t Kp, int64_t N,
                  const uint32_t* __restrict__ P, const void* __restrict__ alpha, int alpha_f16,
                  void* __restrict__ y, int y_dtype, int ntj, int ntiles) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t wl0[kWTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t wl1[kWTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t wl2[kWTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t wl3[kWTileBytes];
    uint8_t* const lds[kRing] = {lds0, lds1, lds2, lds3};
    uint8_t* const wls[kRing] = {wl0, wl1, wl2, wl3};
    const int tile = xcd_tile(blockIdx.x, ntiles);
    if (tile >= ntiles) return;
    const int64_t m0 = int64_t(tile / ntj) * kBM, j0 = int64_t(tile % ntj) * kBJ;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
    const int T = int(Kp / 64);                 // stages, even and >= 2
    constexpr uint32_t kOne = kF16 ? 0x3C003C00u : 0x3F803F80u;

    const uint8_t* src[4];
    dma_plan<true>(reinterpret_cast<const uint8_t*>(xi), Kp * 2, m0, M, tid, src);
    const uint8_t* wsrc = wtile_src(P, j0, N, tid);
    const int wbyte = (64 * wave + r) * 16 + 4 * (g >> 1);   // + 256 f + 8 (s & 1): this lane's word
    // B-operand byte offsets in a stage: token row 16n + r, chunk of MFMA v
    const int rsw = swz16(r);
    const int boff0 = r * 128 + 16 * ((4 * (g >> 1) + (g & 1)) ^ rsw);
    const int boff1 = r * 128 + 16 * ((4 * (g >> 1) + 2 + (g & 1)) ^ rsw);
    const int wshift = 4 * (g & 1);

    auto issue = [&](int s, int B) {            // stage s (clamped: the tail re-reads the last stage)
        const int sc = s < T ? s : T - 1;
        dma_stage(src, int64_t(sc) * 128, lds[B], wave);
        dma16(wsrc + int64_t(sc >> 1) * N * 16, wls[B] + wave * 1024);
    };

    f32x4_t acc[4][8];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[f][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Operands of the next MFMA group, carried between steps: the shifted sign
    // words and the v = 0 B fragments of the stage.
    uint32_t X[4];
    u32x4_t b0[8];
    auto load_head = [&](int s, int B) {
        const int wb = wbyte + 8 * (s & 1);
#pragma unroll
        for (int f = 0; f < 4; ++f) X[f] = *reinterpret_cast<const uint32_t*>(wls[B] + wb + 256 * f) >> wshift;
#pragma unroll
        for (int n = 0; n < 8; ++n) b0[n] = *reinterpret_cast<const u32x4_t*>(lds[B] + n * 2048 + boff0);
    };
    auto mfma_half = [&](int v, const uint32_t (&Xv)[4], const u32x4_t (&b)[8]) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            u32x4_t a;   // (~(X << s) & 0x80008000) | one: sign bits of rows 4u+e, 4u+e+16
            a.x = __builtin_amdgcn_bitop3_b32(Xv[f] << (15 - 8 * v), 0x80008000u, kOne, 0xAE);
            a.y = __builtin_amdgcn_bitop3_b32(Xv[f] << (14 - 8 * v), 0x80008000u, kOne, 0xAE);
            a.z = __builtin_amdgcn_bitop3_b32(Xv[f] << (13 - 8 * v), 0x80008000u, kOne, 0xAE);
            a.w = __builtin_amdgcn_bitop3_b32(Xv[f] << (12 - 8 * v), 0x80008000u, kOne, 0xAE);
#pragma unroll
            for (int n = 0; n < 8; ++n) acc[f][n] = mfma16g<kF16>(a, b[n], acc[f][n]);
        }
    };
    // Step s: the v = 0 half of stage s runs on operands fetched during the
    // previous step while the v = 1 fragments load; then, once every wave has
    // its stage-s reads back and stage s+1 has landed, one barrier frees ring
    // slot s%4 for stage s+4 and the v = 1 half runs while the next stage's
    // head operands load. Each thread issues 5 DMA operations per stage, and
    // stages s+2 and s+3 are in flight behind stage s+1 at the barrier.
    auto step = [&](int s, auto Bc) {
        constexpr int B = decltype(Bc)::value;
        u32x4_t b1[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) b1[n] = *reinterpret_cast<const u32x4_t*>(lds[B] + n * 2048 + boff1);
        uint32_t Xc[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) Xc[f] = X[f];
        mfma_half(0, Xc, b0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt_lgkm0<10>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(s + 4, B);
        load_head(s + 1, (B + 1) % kRing);
        mfma_half(1, Xc, b1);
    };

    issue(0, 0);
    issue(1, 1);
    issue(2, 2);
    issue(3, 3);
    wait_vmcnt<15>();
    __builtin_amdgcn_s_barrier();
    load_head(0, 0);
    int s = 0;
    for (; s + 4 <= T; s += 4) {
        step(s, std::integral_constant<int, 0>{});
        step(s + 1, std::integral_constant<int, 1>{});
        step(s + 2, std::integral_constant<int, 2>{});
        step(s + 3, std::integral_constant<int, 3>{});
    }
    if (s < T) {                                // T even: two stages left
        step(s, std::integral_constant<int, 0>{});
        step(s + 1, std::integral_constant<int, 1>{});
    }
    wait_vmcnt<0>();                            // no LDS DMA may outlive the block

#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int64_t jb = j0 + 64 * wave + 16 * f + 4 * g;
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = jb + i < N ? alpha_at(alpha, alpha_f16, jb + i) : 0.0f;
        const bool full = jb + 4 <= N && (N & 3) == 0;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const int64_t m = m0 + 16 * n + r;
            if (m >= M) continue;
            const int64_t o = m * N + jb;
            const float v0 = al[0] * acc[f][n][0], v1 = al[1] * acc[f][n][1];
            const float v2 = al[2] * acc[f][n][2], v3 = al[3] * acc[f][n][3];
            if (full && y_dtype == kDtF32) {
                *reinterpret_cast<f32x4_t*>(static_cast<float*>(y) + o) = f32x4_t{v0, v1, v2, v3};
            } else if (full) {
                uint16_t h[4];
                if (y_dtype == kDtBF16) {
                    h[0] = f32_to_bf16_rne(v0); h[1] = f32_to_bf16_rne(v1);
                    h[2] = f32_to_bf16_rne(v2); h[3] = f32_to_bf16_rne(v3);
                } else {
                    h[0] = f32_to_f16_rne(v0); h[1] = f32_to_f16_rne(v1);
                    h[2] = f32_to_f16_rne(v2); h[3] = f32_to_f16_rne(v3);
                }
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + o) =
                    uint2{uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16)};
            } else {
                const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (jb + i >= N) continue;
                    if (y_dtype == kDtF32) static_cast<float*>(y)[o + i] = vv[i];
                    else if (y_dtype == kDtBF16) static_cast<uint16_t*>(y)[o + i] = f32_to_bf16_rne(vv[i]);
                    else static_cast<uint16_t*>(y)[o + i] = f32_to_f16_rne(vv[i]);
                }
            }
        }
    }
}

hipError_t launch_w1a16_gemm(const uint16_t* xi, int x_f16, int64_t M, int64_t K, int64_t N, const uint32_t* P,
                             const void* alpha, int alpha_f16, void* y, int y_dtype, hipStream_t s) {
    const int ntj = int((N + kBJ - 1) / kBJ), ntm = int((M + kBM - 1) / kBM);
    const int ntiles = ntj * ntm;
    const unsigned grid = unsigned(xcd_grid(ntiles));
    const int64_t Kp = padded_k(K);
    if (x_f16)
        gemm_w1a16_kernel<true><<<grid, 256, 0, s>>>(xi, M, Kp, N, P, alpha, alpha_f16, y, y_dtype, ntj, ntiles);
    else
        gemm_w1a16_kernel<false><<<grid, 256, 0, s>>>(xi, M, Kp, N, P, alpha, alpha_f16, y, y_dtype, ntj, ntiles);
    return hipGetLastError();
}

// ------------------------------------------------------------------- W1A8 ----
__global__ void __launch_bounds__(256, 2)
gemm_w1a8_kernel(const int8_t* __restrict__ q, const int32_t* __restrict__ rowsum, const float* __restrict__ gamma,
                 const float* __restrict__ beta, float qb, int64_t M, int64_t N, int64_t TQ,
                 const uint32_t* __restrict__ P, float* __restrict__ y, int32_t* __restrict__ acc_opt, int ntj,
                 int ntiles) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t wl0[kWTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t wl1[kWTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t wl2[kWTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t wl3[kWTileBytes];
    uint8_t* const lds[kRing] = {lds0, lds1, lds2, lds3};
    uint8_t* const wls[kRing] = {wl0, wl1, wl2, wl3};
    const int tile = xcd_tile(blockIdx.x, ntiles);
    if (tile >= ntiles) return;
    const int64_t m0 = int64_t(tile / ntj) * kBM, j0 = int64_t(tile % ntj) * kBJ;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
    const int T = int(TQ);                      // one stage per 128-row tile, >= 1

    const uint8_t* src[4];
    dma_plan<false>(reinterpret_cast<const uint8_t*>(q), TQ * 128, m0, M, tid, src);
    const uint8_t* wsrc = wtile_src(P, j0, N, tid);
    const int wbyte = (64 * wave + r) * 16 + 4 * g;          // + 256 f: this lane's word
    const int rsw = swz8(r);
    const int boff0 = r * 128 + 16 * ((2 * g) ^ rsw);
    const int boff1 = r * 128 + 16 * ((2 * g + 1) ^ rsw);

    auto issue = [&](int s, int B) {
        const int sc = s < T ? s : T - 1;
        dma_stage(src, int64_t(sc) * 128, lds[B], wave);
        dma16(wsrc + int64_t(sc) * N * 16, wls[B] + wave * 1024);
    };

    i32x4_t acc[4][8];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[f][n] = i32x4_t{0, 0, 0, 0};

    uint32_t W[4];
    i32x4_t b0[8];
    auto load_head = [&](int B) {
#pragma unroll
        for (int f = 0; f < 4; ++f) W[f] = *reinterpret_cast<const uint32_t*>(wls[B] + wbyte + 256 * f);
#pragma unroll
        for (int n = 0; n < 8; ++n) b0[n] = *reinterpret_cast<const i32x4_t*>(lds[B] + n * 2048 + boff0);
    };
    auto mfma_half = [&](int v, const uint32_t (&Wv)[4], const i32x4_t (&b)[8]) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const uint32_t w = Wv[f];
            i32x4_t a;
            a.x = int((w >> (4 * v + 0)) & 0x01010101u);
            a.y = int((w >> (4 * v + 1)) & 0x01010101u);
            a.z = int((w >> (4 * v + 2)) & 0x01010101u);
            a.w = int((w >> (4 * v + 3)) & 0x01010101u);
#pragma unroll
            for (int n = 0; n < 8; ++n)
                acc[f][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[n], acc[f][n], 0, 0, 0);
        }
    };
    // Same step structure as the W1A16 kernel.
    auto step = [&](int s, auto Bc) {
        constexpr int B = decltype(Bc)::value;
        i32x4_t b1[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) b1[n] = *reinterpret_cast<const i32x4_t*>(lds[B] + n * 2048 + boff1);
        uint32_t Wc[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) Wc[f] = W[f];
        mfma_half(0, Wc, b0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt_lgkm0<10>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(s + 4, B);
        load_head((B + 1) % kRing);
        mfma_half(1, Wc, b1);
    };

    issue(0, 0);
    issue(1, 1);
    issue(2, 2);
    issue(3, 3);
    wait_vmcnt<15>();
    __builtin_amdgcn_s_barrier();
    load_head(0);
    int s = 0;
    for (; s + 4 <= T; s += 4) {
        step(s, std::integral_constant<int, 0>{});
        step(s + 1, std::integral_constant<int, 1>{});
        step(s + 2, std::integral_constant<int, 2>{});
        step(s + 3, std::integral_constant<int, 3>{});
    }
    if (s < T) step(s, std::integral_constant<int, 0>{});
    if (s + 1 < T) step(s + 1, std::integral_constant<int, 1>{});
    if (s + 2 < T) step(s + 2, std::integral_constant<int, 2>{});
    wait_vmcnt<0>();

    const float scale = (beta[0] * gamma[0]) / qb;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int64_t jb = j0 + 64 * wave + 16 * f + 4 * g;
        const bool full = jb + 4 <= N && (N & 3) == 0;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const int64_t m = m0 + 16 * n + r;
            if (m >= M) continue;
            const int32_t rs = rowsum[m];
            const int64_t o = m * N + jb;
            i32x4_t a;
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = 2 * acc[f][n][i] - rs;
            if (full) {
                *reinterpret_cast<f32x4_t*>(y + o) =
                    f32x4_t{float(a[0]) * scale, float(a[1]) * scale, float(a[2]) * scale, float(a[3]) * scale};
                if (acc_opt) *reinterpret_cast<i32x4_t*>(acc_opt + o) = a;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (jb + i >= N) continue;
                    y[o + i] = float(a[i]) * scale;
                    if (acc_opt) acc_opt[o + i] = a[i];
                }
            }
        }
    }
}

hipError_t launch_w1a8_gemm(const int8_t* q, const int32_t* rowsum, const float* gamma, const float* beta, float qb,
                            int64_t M, int64_t K, int64_t N, const uint32_t* P, float* y, int32_t* acc_opt,
                            hipStream_t s) {
    const int ntj = int((N + kBJ - 1) / kBJ), ntm = int((M + kBM - 1) / kBM);
    const int ntiles = ntj * ntm;
    gemm_w1a8_kernel<<<unsigned(xcd_grid(ntiles)), 256, 0, s>>>(q, rowsum, gamma, beta, qb, M, N, tiles_per_col(K),
                                                                  P, y, acc_opt, ntj, ntiles);
    return hipGetLastError();
}

}  // namespace bgb
