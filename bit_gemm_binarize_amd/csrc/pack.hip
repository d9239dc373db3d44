// Weight conversion: sign binarization + 1-bit packing, with the scales.
//
// FBI-linear (FBI-LLM news rewrite, paragraph introducing FBI-linear): sign of
// W (ties to -1 as in "BitNet b1.58: 1bit LLM时代", section 一, eq. (2)) and a
// per-output-column scale alpha_j = mean_i |W_ij|.
// BitNet (same blog, eq. (1)-(3), (8)): sign of W - c with c = mean(W), and
// beta = mean |W|.
//
// BitNet b1.58 (same blog, section 二, eq. (9)-(11)): ternary weights
// RoundClip(W / (gamma_w + eps), -1, 1) with gamma_w = mean |W|, stored as two
// sign planes in the same format (the +1 plane, then the -1 plane).
//
// All are single passes over fp32 W after the reductions (HBM-bound: 4 bytes
// read per weight, 1/8 or 1/4 byte written). Sums are fp64 over fixed partitions combined in a fixed
// order, so every output is reproducible bit for bit.
#include "bgb_device.hpp"
#include "bgb_internal.hpp"

namespace bgb {

// One thread per (128-row tile, column): reads W[128 tq .. 128 tq + 127][j]
// (a wave covers 64 adjacent columns, 256 contiguous bytes per row), builds
// the column's 4 words and stores them as one 16-byte tile.
template <bool kBitnet>
__global__ void __launch_bounds__(256)
pack_signs_kernel(const float* __restrict__ W, int64_t K, int64_t N, uint32_t* __restrict__ P,
                  double* __restrict__ colsum, const float* __restrict__ centre) {
    const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t tq = blockIdx.y;
    if (j >= N) return;
    const int64_t T = K / 32;
    // W > c exactly (BitNet): on order keys, false when either side is NaN;
    // the centre's key and NaN test are computed once
    const float c = kBitnet ? centre[0] : 0.0f;
    const uint32_t kc = f32_order_key(c);
    const bool cnan = f32_is_nan(c);
    uint32_t words[4];
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int64_t t = tq * 4 + w;
        uint32_t word = 0;
        if (t < T) {                                   // uniform: t depends on the block only
            // the word's 32 loads are issued before any of them is used
            const float* col = W + (32 * t) * N + j;
            float v[32];
#pragma unroll
            for (int b = 0; b < 32; ++b) v[b] = __builtin_nontemporal_load(col + int64_t(b) * N);
#pragma unroll
            for (int b = 0; b < 32; ++b) {
                const bool pos = kBitnet ? (!f32_is_nan(v[b]) & !cnan & (f32_order_key(v[b]) > kc))
                                         : f32_gt_zero(v[b]);
                word |= uint32_t(pos) << b;
                if (!kBitnet) s += fabs(double(v[b]));
            }
        }
        words[w] = word;
    }
    u32x4_t out = {words[0], words[1], words[2], words[3]};
    *reinterpret_cast<u32x4_t*>(P + (tq * N + j) * 4) = out;
    if (!kBitnet) colsum[tq * N + j] = s;
}

// Ternary planes: one thread per (128-row tile, column), as above. The
// quotient W / (gamma_w + eps) is a correctly rounded fp32 division; round()
// is to nearest even. Plane 0 (+1) at P, plane 1 (-1) at P + TQ N 4 words.
__global__ void __launch_bounds__(256)
pack_ternary_kernel(const float* __restrict__ W, int64_t K, int64_t N, uint32_t* __restrict__ P,
                    const float* __restrict__ gamma_w) {
    const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t tq = blockIdx.y;
    if (j >= N) return;
    const int64_t T = K / 32, TQ = gridDim.y;
    const float den = gamma_w[0] + kTernaryEps;
    uint32_t pos[4], neg[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int64_t t = tq * 4 + w;
        uint32_t wp = 0, wn = 0;
        if (t < T) {                                   // uniform: t depends on the block only
            const float* col = W + (32 * t) * N + j;
            float v[32];                               // the word's 32 loads in flight together
#pragma unroll
            for (int b = 0; b < 32; ++b) v[b] = __builtin_nontemporal_load(col + int64_t(b) * N);
#pragma unroll
            for (int b = 0; b < 32; ++b) {
                const float r = __builtin_rintf(v[b] / den);
                wp |= uint32_t(r >= 1.0f) << b;
                wn |= uint32_t(r <= -1.0f) << b;
            }
        }
        pos[w] = wp;
        neg[w] = wn;
    }
    *reinterpret_cast<u32x4_t*>(P + (tq * N + j) * 4) = u32x4_t{pos[0], pos[1], pos[2], pos[3]};
    *reinterpret_cast<u32x4_t*>(P + (TQ * N + tq * N + j) * 4) = u32x4_t{neg[0], neg[1], neg[2], neg[3]};
}

// alpha_j = fl32((sum over tiles of the tile sums, in tile order) / K).
__global__ void __launch_bounds__(256)
fbi_alpha_kernel(const double* __restrict__ colsum, int64_t TQ, int64_t N, int64_t K,
                 void* __restrict__ alpha, int alpha_f16) {
    const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (j >= N) return;
    double s = 0.0;
    for (int64_t t0 = 0; t0 < TQ; t0 += 8) {       // 8 loads in flight, added in tile order
        double v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = colsum[(t0 + q < TQ ? t0 + q : TQ - 1) * N + j];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (t0 + q < TQ) s += v[q];
    }
    const float a = float(s / double(K));
    if (alpha_f16) reinterpret_cast<uint16_t*>(alpha)[j] = f32_to_f16_rne(a);
    else reinterpret_cast<float*>(alpha)[j] = a;
}

// Partial (sum W, sum |W|) per block over a fixed grid-stride partition.
__global__ void __launch_bounds__(256)
bitnet_reduce_kernel(const float* __restrict__ W, int64_t n, double* __restrict__ partial) {
    __shared__ double scratch[4];
    double s = 0.0, a = 0.0;
    const int64_t stride = int64_t(gridDim.x) * 256 * 4;
    for (int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4; i < n; i += stride) {
        typedef float f32x4v __attribute__((ext_vector_type(4)));
        const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(W + i));
        s += double(v.x); s += double(v.y); s += double(v.z); s += double(v.w);
        a += fabs(double(v.x)); a += fabs(double(v.y)); a += fabs(double(v.z)); a += fabs(double(v.w));
    }
    s = block_sum<256>(s, scratch);
    a = block_sum<256>(a, scratch);
    if (threadIdx.x == 0) {
        partial[2 * blockIdx.x] = s;
        partial[2 * blockIdx.x + 1] = a;
    }
}

// c = fl32(S / (K N)), beta = fl32(A / (K N)); one block.
__global__ void __launch_bounds__(256)
bitnet_finalize_kernel(const double* __restrict__ partial, int nblocks, double count,
                       float* __restrict__ centre, float* __restrict__ beta) {
    __shared__ double scratch[4];
    double s = 0.0, a = 0.0;
    for (int b = threadIdx.x; b < nblocks; b += 256) {
        s += partial[2 * b];
        a += partial[2 * b + 1];
    }
    s = block_sum<256>(s, scratch);
    a = block_sum<256>(a, scratch);
    if (threadIdx.x == 0) {
        centre[0] = float(s / count);
        beta[0] = float(a / count);
    }
}

hipError_t launch_pack(const float* W, int64_t K, int64_t N, int mode, uint32_t* P,
                       void* alpha, int alpha_f16, float* beta, float* centre,
                       void* ws, hipStream_t s) {
    const int64_t TQ = tiles_per_col(K);
    const dim3 grid(unsigned((N + 255) / 256), unsigned(TQ));
    if (mode == 0) {
        double* colsum = reinterpret_cast<double*>(static_cast<char*>(ws) + PackFbiWs::make(K, N).colsum);
        pack_signs_kernel<false><<<grid, 256, 0, s>>>(W, K, N, P, colsum, nullptr);
        fbi_alpha_kernel<<<unsigned((N + 255) / 256), 256, 0, s>>>(colsum, TQ, N, K, alpha, alpha_f16);
    } else {
        const PackBitnetWs lay = PackBitnetWs::make();
        double* partial = reinterpret_cast<double*>(static_cast<char*>(ws) + lay.partial);
        float* c = centre ? centre : reinterpret_cast<float*>(static_cast<char*>(ws) + lay.scratch);
        const int64_t n = K * N;
        int64_t nb = (n + 256 * 4 - 1) / (256 * 4);
        if (nb > kBitnetReduceBlocks) nb = kBitnetReduceBlocks;
        bitnet_reduce_kernel<<<unsigned(nb), 256, 0, s>>>(W, n, partial);
        bitnet_finalize_kernel<<<1, 256, 0, s>>>(partial, int(nb), double(K) * double(N), c, beta);
        if (mode == 1) pack_signs_kernel<true><<<grid, 256, 0, s>>>(W, K, N, P, nullptr, c);
        else pack_ternary_kernel<<<grid, 256, 0, s>>>(W, K, N, P, beta);    // beta = mean |W| = gamma_w
    }
    return hipGetLastError();
}

}  // namespace bgb
