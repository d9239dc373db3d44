// Ceiling microbenchmarks for gfx950: what the hardware gives this code at
// the clock it holds, against which the product kernels are read. Measurement
// tools only: nothing here is on the product's compute path, and the product
// library does not link it. Declarations in include/bgb_ceilings.h.
//
//   ceil_stream_read  grid-stride 16-byte loads over a buffer (HBM or MALL
//                     bandwidth at a given size per launch)
//   ceil_empty        an empty kernel of a given launch shape (launch cost)
//   ceil_mfma_bf16    register-only v_mfma_f32_16x16x32_bf16 chains
//   ceil_mfma_i8      register-only v_mfma_i32_16x16x64_i8 chains
// The MFMA loops take their operands from a buffer of random values: the
// matrix cores' power, hence the clock they sustain, depends on how many
// operand bits toggle.
#include "../../include/bgb_ceilings.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

thread_local int g_err = 0;

int done(hipError_t e) {
    if (e != hipSuccess) {
        g_err = int(e);
        return -3;
    }
    return 0;
}

// Each thread XORs the 16-byte words it reads; the sum is stored only when a
// flag the host never sets is set, so the loads cannot be dropped.
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ p, size_t n, int flag,
                                                          uint32_t* __restrict__ sink) {
    u32x4 a = {0u, 0u, 0u, 0u};
    const size_t stride = size_t(gridDim.x) * blockDim.x;
    size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + 7 * stride < n; i += 8 * stride) {           // eight 16-byte loads in flight per lane
        u32x4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
        for (int k = 0; k < 8; ++k) a ^= v[k];
    }
    for (; i < n; i += stride) a ^= p[i];
    if (flag) sink[blockIdx.x * blockDim.x + threadIdx.x] = a.x ^ a.y ^ a.z ^ a.w;
}

__global__ void empty_kernel() {}

// Eight independent accumulator chains per wave, written as one asm block so
// that each chain keeps its own registers (as builtins, the compiler rotated
// the chains through overlapping register copies, which serialised them).
#define BGB_CEIL_MFMA8(OP)                                                                                    \
    asm volatile(OP " %0, %8, %9, %0\n\t" OP " %1, %8, %9, %1\n\t" OP " %2, %8, %9, %2\n\t" OP              \
                    " %3, %8, %9, %3\n\t" OP " %4, %8, %9, %4\n\t" OP " %5, %8, %9, %5\n\t" OP              \
                    " %6, %8, %9, %6\n\t" OP " %7, %8, %9, %7\n\t"                                           \
                 : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3), "+a"(c4), "+a"(c5), "+a"(c6), "+a"(c7)            \
                 : "v"(a), "v"(b))

__global__ void __launch_bounds__(256) mfma_bf16_kernel(const u32x4* __restrict__ src, int iters, int flag,
                                                        float* __restrict__ sink) {
    const int t = (blockIdx.x * blockDim.x + threadIdx.x) & 4095;
    const u32x4 a = src[t], b = src[4096 + t];
    f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
    for (int it = 0; it < iters; ++it) BGB_CEIL_MFMA8("v_mfma_f32_16x16x32_bf16");
    const f32x4 s = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
    if (flag) sink[blockIdx.x * blockDim.x + threadIdx.x] = s.x + s.y + s.z + s.w;
}

__global__ void __launch_bounds__(256) mfma_i8_kernel(const u32x4* __restrict__ src, int iters, int flag,
                                                      int* __restrict__ sink) {
    const int t = (blockIdx.x * blockDim.x + threadIdx.x) & 4095;
    const u32x4 a = src[t], b = src[4096 + t];
    i32x4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
    for (int it = 0; it < iters; ++it) BGB_CEIL_MFMA8("v_mfma_i32_16x16x64_i8");
    const i32x4 s = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
    if (flag) sink[blockIdx.x * blockDim.x + threadIdx.x] = s.x + s.y + s.z + s.w;
}

#undef BGB_CEIL_MFMA8

}  // namespace

extern "C" {

int ceil_stream_read(const void* buf, size_t bytes, int blocks, void* sink, void* stream) {
    if (!buf || (reinterpret_cast<uintptr_t>(buf) & 15u) || bytes % 16 || blocks <= 0 || blocks > 65536)
        return -1;
    stream_read_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4*>(buf), bytes / 16, 0, static_cast<uint32_t*>(sink));
    return done(hipGetLastError());
}

int ceil_empty(int blocks, int threads, void* stream) {
    if (blocks <= 0 || threads <= 0 || threads > 1024) return -1;
    empty_kernel<<<blocks, threads, 0, static_cast<hipStream_t>(stream)>>>();
    return done(hipGetLastError());
}

int ceil_mfma_bf16(const void* random_bits, int blocks, int iters, void* sink, void* stream) {
    if (!random_bits || (reinterpret_cast<uintptr_t>(random_bits) & 15u) || blocks <= 0 || iters <= 0) return -1;
    mfma_bf16_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4*>(random_bits), iters, 0, static_cast<float*>(sink));
    return done(hipGetLastError());
}

int ceil_mfma_i8(const void* random_bits, int blocks, int iters, void* sink, void* stream) {
    if (!random_bits || (reinterpret_cast<uintptr_t>(random_bits) & 15u) || blocks <= 0 || iters <= 0) return -1;
    mfma_i8_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4*>(random_bits), iters, 0, static_cast<int*>(sink));
    return done(hipGetLastError());
}

int ceil_last_hip_error(void) { return g_err; }

}  // extern "C"
