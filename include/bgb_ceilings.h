/*
 * bgb_ceilings.h -- ceiling microbenchmarks for gfx950 (libbgb_ceilings.so).
 *
 * Measurement tools, not part of the binarized-linear boundary in bgb.h:
 * they measure what the GPU gives simple code at the clock it holds, so that
 * the product kernels' rates can be read as a fraction of an achievable
 * ceiling as well as of the vendor's peak figures.
 *
 * All pointers are device pointers, 16-byte aligned, owned by the caller;
 * calls are asynchronous on `stream` (a hipStream_t, NULL = null stream).
 * Return 0, -1 for a bad argument (nothing launched) or -3 for a failed
 * launch (ceil_last_hip_error() has the hipError_t).
 */
#ifndef BGB_CEILINGS_H
#define BGB_CEILINGS_H
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16) of `buf` once with 16-byte loads, grid-
 * stride over `blocks` blocks of 256 threads. `sink` (blocks * 256 uint32)
 * is never written in practice; it keeps the loads alive. */
int ceil_stream_read(const void* buf, size_t bytes, int blocks, void* sink, void* stream);

/* An empty kernel of `blocks` x `threads`: the launch cost alone. */
int ceil_empty(int blocks, int threads, void* stream);

/* `iters` x 8 independent v_mfma_f32_16x16x32_bf16 per wave (16384 flop
 * each), `blocks` blocks of 256 threads, operands from `random_bits`
 * (at least 8192 x 16 bytes; finite bf16 values). `sink`: blocks * 256 floats, kept alive. */
int ceil_mfma_bf16(const void* random_bits, int blocks, int iters, void* sink, void* stream);

/* The same with v_mfma_i32_16x16x64_i8 (32768 ops each); `sink`: int32. */
int ceil_mfma_i8(const void* random_bits, int blocks, int iters, void* sink, void* stream);

int ceil_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif
