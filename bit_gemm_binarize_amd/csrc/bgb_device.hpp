// Device-side helpers shared by the kernels (gfx950, wave64).
#pragma once
#include <type_traits>

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#define BGB_DEV __device__ __forceinline__

namespace bgb {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

enum { kDtF32 = 0, kDtF16 = 1, kDtBF16 = 2 };

// 16-bit float formats <-> float (round to nearest even on the way down).
BGB_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
BGB_DEV float f16_to_f32(uint16_t h) { return __half2float(__ushort_as_half(h)); }
BGB_DEV uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);   // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}
BGB_DEV uint16_t f32_to_f16_rne(float f) { return __half_as_ushort(__float2half_rn(f)); }

// Exact "a > b" for fp32 independent of the denormal mode: NaN compares
// false, +0 == -0, subnormals keep their order.
BGB_DEV uint32_t f32_order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) == 0) u = 0;                    // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
BGB_DEV bool f32_is_nan(float v) { return (__float_as_uint(v) & 0x7fffffffu) > 0x7f800000u; }
BGB_DEV bool f32_gt_exact(float a, float b) {
    if (f32_is_nan(a) || f32_is_nan(b)) return false;
    return f32_order_key(a) > f32_order_key(b);
}
// a > 0 on the bit pattern: positive subnormals and +inf are > 0; zeros and NaN are not.
BGB_DEV bool f32_gt_zero(float a) {
    uint32_t u = __float_as_uint(a);
    return int32_t(u) > 0 && u <= 0x7f800000u;
}

// ---- wave / block reductions (fixed trees -> deterministic) -----------------
BGB_DEV double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
BGB_DEV float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
BGB_DEV int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Wave reductions on the DPP network (gfx9 row/bank controls): quad swaps,
// half-row and row mirrors, then row_bcast15 / row_bcast31 fold the four rows
// of 16 lanes; the total lands in lane 63. Lanes outside a broadcast's row
// mask add the identity (0). Fixed order, so the result is reproducible.
template <int CTRL, int ROWMASK>
BGB_DEV int dpp_i32(int v) {
    // all rows enabled (the quad swaps and mirrors read a valid lane for every
    // lane): no old value to keep; else the disabled rows keep 0
    if constexpr (ROWMASK == 0xF) return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
    else return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWMASK, 0xF, false);
}
template <int CTRL, int ROWMASK>
BGB_DEV double dpp_f64(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = dpp_i32<CTRL, ROWMASK>(int(b & 0xffffffffll));
    const int hi = dpp_i32<CTRL, ROWMASK>(int(b >> 32));
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}
template <int CTRL, int ROWMASK>
BGB_DEV float dpp_f32(float v) {
    return __int_as_float(dpp_i32<CTRL, ROWMASK>(__float_as_int(v)));
}
// Sum over the 64 lanes, valid in lane 63.
BGB_DEV double wave_sum63(double v) {
    v += dpp_f64<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    v += dpp_f64<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    v += dpp_f64<0x141, 0xF>(v);   // row_half_mirror
    v += dpp_f64<0x140, 0xF>(v);   // row_mirror
    v += dpp_f64<0x142, 0xA>(v);   // row_bcast15 into rows 1, 3
    v += dpp_f64<0x143, 0xC>(v);   // row_bcast31 into rows 2, 3
    return v;
}
// Sum of n (a power of two) values in a fixed pairwise tree order.
template <int n>
BGB_DEV double tree_sum(const double* a) {
    if constexpr (n == 1) return a[0];
    else return tree_sum<n / 2>(a) + tree_sum<n / 2>(a + n / 2);
}
BGB_DEV int wave_sum63_i(int v) {
    v += dpp_i32<0xB1, 0xF>(v);
    v += dpp_i32<0x4E, 0xF>(v);
    v += dpp_i32<0x141, 0xF>(v);
    v += dpp_i32<0x140, 0xF>(v);
    v += dpp_i32<0x142, 0xA>(v);
    v += dpp_i32<0x143, 0xC>(v);
    return v;
}
// Integer code of a quantizer input v: truncation toward zero, or (rne)
// rounding to nearest, ties to even; clamped to +-qmax either way (a no-op for
// truncation of a value already clipped to +-(Q_b - eps)).
BGB_DEV int round_code(float v, bool rne, int qmax) {
    const int c = rne ? int(__builtin_rintf(v)) : int(v);
    return c > qmax ? qmax : (c < -qmax ? -qmax : c);
}
// Whether a fast quotient u, within 1.5 ulp of the exact one, lies so close to
// a point where the code changes (a nonzero integer for truncation, a
// half-integer for rounding) that the exact division has to decide.
BGB_DEV bool code_near_boundary(float u, bool rne) {
    const float d = __builtin_fabsf(u - __builtin_rintf(u));
    return (rne ? __builtin_fabsf(d - 0.5f) : d) < __builtin_fabsf(u) * 0x1p-20f;
}

// Order-preserving map of fp32 bit patterns onto uint32: for non-NaN x < y,
// key(x) < key(y) (-0 sorts just below +0). Negative values are complemented,
// non-negative ones get the top bit set.
BGB_DEV uint32_t f32_sort_key(float x) {
    const uint32_t b = __float_as_uint(x);
    return b ^ (uint32_t(int32_t(b) >> 31) | 0x80000000u);
}
BGB_DEV float f32_from_sort_key(uint32_t k) {
    return __uint_as_float(k ^ (~uint32_t(int32_t(k) >> 31) | 0x80000000u));
}

// Unsigned max over the 64 lanes, valid in lane 63 (0 is the identity).
BGB_DEV uint32_t wave_umax63(uint32_t v) {
    v = max(v, uint32_t(dpp_i32<0xB1, 0xF>(int(v))));
    v = max(v, uint32_t(dpp_i32<0x4E, 0xF>(int(v))));
    v = max(v, uint32_t(dpp_i32<0x141, 0xF>(int(v))));
    v = max(v, uint32_t(dpp_i32<0x140, 0xF>(int(v))));
    v = max(v, uint32_t(dpp_i32<0x142, 0xA>(int(v))));
    v = max(v, uint32_t(dpp_i32<0x143, 0xC>(int(v))));
    return v;
}
// Max of non-negative values over the 64 lanes, valid in lane 63.
BGB_DEV float wave_max63_nonneg(float v) {
    v = fmaxf(v, dpp_f32<0xB1, 0xF>(v));
    v = fmaxf(v, dpp_f32<0x4E, 0xF>(v));
    v = fmaxf(v, dpp_f32<0x141, 0xF>(v));
    v = fmaxf(v, dpp_f32<0x140, 0xF>(v));
    v = fmaxf(v, dpp_f32<0x142, 0xA>(v));
    v = fmaxf(v, dpp_f32<0x143, 0xC>(v));
    return v;
}
// Max / min over the 64 lanes (any values), valid in lane 63; disabled rows of
// the broadcast steps contribute the identity (-inf / +inf).
template <int CTRL, int ROWMASK>
BGB_DEV float dpp_f32_id(float v, float id) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(id), __float_as_int(v), CTRL, ROWMASK, 0xF,
                                                      false));
}
BGB_DEV float wave_max63(float v) {
    const float id = -__builtin_inff();
    v = fmaxf(v, dpp_f32_id<0xB1, 0xF>(v, id));
    v = fmaxf(v, dpp_f32_id<0x4E, 0xF>(v, id));
    v = fmaxf(v, dpp_f32_id<0x141, 0xF>(v, id));
    v = fmaxf(v, dpp_f32_id<0x140, 0xF>(v, id));
    v = fmaxf(v, dpp_f32_id<0x142, 0xA>(v, id));
    v = fmaxf(v, dpp_f32_id<0x143, 0xC>(v, id));
    return v;
}
BGB_DEV float wave_min63(float v) {
    const float id = __builtin_inff();
    v = fminf(v, dpp_f32_id<0xB1, 0xF>(v, id));
    v = fminf(v, dpp_f32_id<0x4E, 0xF>(v, id));
    v = fminf(v, dpp_f32_id<0x141, 0xF>(v, id));
    v = fminf(v, dpp_f32_id<0x140, 0xF>(v, id));
    v = fminf(v, dpp_f32_id<0x142, 0xA>(v, id));
    v = fminf(v, dpp_f32_id<0x143, 0xC>(v, id));
    return v;
}
// One block pass reducing (sum, max, min) together; `scr` holds NT/64 entries.
struct SumMaxMin { double s; float mx, mn; };
template <int NT>
BGB_DEV SumMaxMin block_sum_max_min(double s, float mx, float mn, SumMaxMin* scr) {
    s = wave_sum63(s);
    mx = wave_max63(mx);
    mn = wave_min63(mn);
    __syncthreads();
    if ((threadIdx.x & 63) == 63) scr[threadIdx.x >> 6] = SumMaxMin{s, mx, mn};
    __syncthreads();
    SumMaxMin t = scr[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) {
        t.s += scr[i].s;
        t.mx = fmaxf(t.mx, scr[i].mx);
        t.mn = fminf(t.mn, scr[i].mn);
    }
    return t;
}

// Block (NT threads) sum / max through the DPP wave reductions: lane 63 of
// each wave parks its value in `scratch`, then every thread adds the NT/64
// values in wave order. Contains two barriers.
template <int NT>
BGB_DEV double block_sum_dpp(double v, double* scratch) {
    v = wave_sum63(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 63) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    double t = scratch[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) t += scratch[i];
    return t;
}
template <int NT>
BGB_DEV float block_max_dpp(float v, float* scratch) {
    v = wave_max63_nonneg(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 63) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = scratch[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) t = fmaxf(t, scratch[i]);
    return t;
}

// Block-wide reductions; `scratch` must hold blockDim.x/64 entries. All
// threads get the result. Contains __syncthreads().
template <int NT>
BGB_DEV double block_sum(double v, double* scratch) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[w] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) t += scratch[i];
    return t;
}
template <int NT>
BGB_DEV float block_max(float v, float* scratch) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[w] = v;
    __syncthreads();
    float t = scratch[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) t = fmaxf(t, scratch[i]);
    return t;
}
template <int NT>
BGB_DEV int block_sum_i(int v, int* scratch) {
    v = wave_sum_i(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[w] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) t += scratch[i];
    return t;
}

// Rank the tiles so that each of the 8 XCDs (block b runs on XCD b % 8)
// works through one contiguous range of tiles. Launch 8 * ceil(n/8) blocks;
// a block whose tile is >= n has nothing to do.
BGB_DEV int xcd_tile(int b, int n) {
    const int per = (n + 7) / 8;
    return (b % 8) * per + b / 8;
}
inline int xcd_grid(int n) { return 8 * ((n + 7) / 8); }

}  // namespace bgb
