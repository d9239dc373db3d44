// bitlinear_w1a8_noalloc: bitlinear_w1a8 with its workspace in a static
// device array instead of a caller's buffer, for callers that cannot allocate
// (code under HIP graph capture, serving loops, harnesses that forbid
// hipMalloc). The declaration and contract are in include/bgb.h.
//
// The array lives in this file's code object: every GPU the library runs on
// holds its own copy, at its own address, until the process ends. Host code
// never uses the array's name as an address (on the host it is only a
// stand-in symbol); the device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and is what the kernels receive.
#include "../../include/bgb.h"
#include "bgb_internal.hpp"

#include <atomic>
#include <mutex>
#include <stdint.h>

static constexpr size_t kScratchBytes = size_t(BGB_NOALLOC_SCRATCH_BYTES);

// The workspace of bitlinear_w1a8_noalloc (one copy per GPU).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// The device address of `scratch` on the current device (looked up once per
// device); nullptr and the HIP error in *err when the lookup fails.
void* scratch_on_current_device(hipError_t* err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess || !p) {
            if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" {

size_t bgb_noalloc_scratch_bytes(void) { return kScratchBytes; }

int bitlinear_w1a8_noalloc(const void* x, int x_dtype, int64_t M, int64_t K, int64_t N, const uint32_t* P,
                           const float* beta, const bgb_quant_params* qp, float* y, int8_t* xq_opt,
                           float* gamma_opt, int32_t* acc_opt, void* stream) {
    // the size check needs no device: a call too large for the array is
    // rejected before anything touches the GPU
    const size_t need = bgb_workspace_bytes(BGB_OP_BITLINEAR, M, K, N);
    if (need > kScratchBytes) return BGB_ESCRATCH;
    if (M == 0 || N == 0)                         // empty: validated, nothing launched, no device needed
        return bitlinear_w1a8(x, x_dtype, M, K, N, P, beta, qp, y, xq_opt, gamma_opt, acc_opt, nullptr, 0,
                              stream);
    hipError_t err = hipSuccess;
    void* ws = scratch_on_current_device(&err);
    if (!ws) {
        bgb::set_last_hip_error(int(err));
        return BGB_EHIP;
    }
    return bitlinear_w1a8(x, x_dtype, M, K, N, P, beta, qp, y, xq_opt, gamma_opt, acc_opt, ws, kScratchBytes,
                          stream);
}

}  // extern "C"
