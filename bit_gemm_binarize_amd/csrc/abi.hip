// C ABI of libbgb.so: argument validation, workspace carving, dispatch on M.
// The declarations and the full contract are in include/bgb.h.
#include "../../include/bgb.h"
#include "bgb_internal.hpp"

#include <stdint.h>

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxDim = int64_t(1) << 24;
constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;

// Shared shape rules; M may be 0 (empty), N may be 0 (empty).
int check_shape(int64_t M, int64_t K, int64_t N) {
    if (K <= 0 || (K % 32) != 0 || K > bgb::kMaxK) return BGB_EINVAL;
    if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim) return BGB_EINVAL;
    if (M * K > kMaxElems || K * N > kMaxElems || M * N > kMaxElems) return BGB_EINVAL;
    return BGB_OK;
}

int finish(hipError_t e) {
    if (e != hipSuccess) {
        g_last_hip_error = int(e);
        return BGB_EHIP;
    }
    return BGB_OK;
}

char* carve(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

}  // namespace

namespace bgb {
void set_last_hip_error(int e) { g_last_hip_error = e; }
}  // namespace bgb

extern "C" {

size_t bgb_packed_bytes(int64_t K, int64_t N) {
    if (K <= 0 || (K % 32) != 0 || N < 0) return 0;
    return size_t(bgb::tiles_per_col(K)) * size_t(N) * 16u;
}

size_t bgb_workspace_bytes(int op, int64_t M, int64_t K, int64_t N) {
    if (K <= 0 || (K % 32) != 0 || M < 0 || N < 0) return 0;
    switch (op) {
        case BGB_OP_PACK_FBI: return bgb::PackFbiWs::make(K, N).total;
        case BGB_OP_PACK_BITNET: return bgb::PackBitnetWs::make().total;
        case BGB_OP_FBI_LINEAR: return bgb::FbiLinearWs::make(M, K, N).total;
        case BGB_OP_BITLINEAR: return bgb::BitlinearWs::make(M, K, N).total;
        case BGB_OP_BITLINEAR158: return bgb::BitlinearWs::make(M, K, N, true).total;
        case BGB_OP_FBI_BACKWARD: return bgb::FbiBackwardWs::make(M, K, N).total;
        default: return 0;
    }
}

int binarize_pack(const float* W, int64_t K, int64_t N, int mode, uint32_t* P, void* alpha, int alpha_dtype,
                  float* beta, float* centre, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(0, K, N);
    if (rc) return rc;
    if (mode != BGB_MODE_FBI && mode != BGB_MODE_BITNET && mode != BGB_MODE_TERNARY) return BGB_EUNSUPPORTED;
    if (mode == BGB_MODE_FBI && alpha_dtype != BGB_F32 && alpha_dtype != BGB_F16) return BGB_EUNSUPPORTED;
    if (N == 0) return BGB_OK;                    // empty: nothing is read or written
    if (!W || !P || !aligned16(W) || !aligned16(P)) return BGB_EINVAL;
    if (mode == BGB_MODE_FBI) {
        if (!alpha || !aligned16(alpha)) return BGB_EINVAL;
    } else if (mode == BGB_MODE_BITNET) {
        if (!beta || !centre || !aligned16(beta) || !aligned16(centre)) return BGB_EINVAL;
    } else {                                      // ternary: centre optional
        if (!beta || !aligned16(beta) || (centre && !aligned16(centre))) return BGB_EINVAL;
    }
    const int op = mode == BGB_MODE_FBI ? BGB_OP_PACK_FBI : BGB_OP_PACK_BITNET;
    const size_t need = bgb_workspace_bytes(op, 0, K, N);
    if (need && (!ws || ws_bytes < need || !aligned16(ws))) return BGB_EINVAL;
    return finish(bgb::launch_pack(W, K, N, mode, P, alpha, alpha_dtype == BGB_F16, beta, centre, ws,
                                   static_cast<hipStream_t>(stream)));
}

// Argument checks of one FBI-linear (the dtypes are checked by the caller):
// BGB_OK with *empty set when nothing is to be done.
static int fbi_check(const void* x, int64_t M, int64_t K, int64_t N, const uint32_t* P, const void* alpha,
                     const void* y, bool* empty) {
    int rc = check_shape(M, K, N);
    if (rc) return rc;
    *empty = M == 0 || N == 0;
    if (*empty) return BGB_OK;                    // empty: nothing is read or written
    if (!x || !P || !alpha || !y) return BGB_EINVAL;
    if (!aligned16(x) || !aligned16(P) || !aligned16(alpha) || !aligned16(y)) return BGB_EINVAL;
    return BGB_OK;
}

static int fbi_dtypes(int x_dtype, int alpha_dtype, int y_dtype) {
    if (x_dtype != BGB_BF16 && x_dtype != BGB_F16) return BGB_EUNSUPPORTED;
    if (alpha_dtype != BGB_F32 && alpha_dtype != BGB_F16) return BGB_EUNSUPPORTED;
    if (y_dtype != BGB_F32 && y_dtype != BGB_BF16 && y_dtype != BGB_F16) return BGB_EUNSUPPORTED;
    return BGB_OK;
}

// The launches of one checked, non-empty FBI-linear (ws already checked).
static int fbi_run(const void* x, int x_dtype, int64_t M, int64_t K, int64_t N, const uint32_t* P,
                   const void* alpha, int alpha_dtype, void* y, int y_dtype, void* ws, hipStream_t s) {
    const bgb::FbiLinearWs lay = bgb::FbiLinearWs::make(M, K, N);
    const int x_f16 = x_dtype == BGB_F16;
    const int a_f16 = alpha_dtype == BGB_F16;
    const int ydt = y_dtype == BGB_F32 ? 0 : (y_dtype == BGB_F16 ? 1 : 2);
    if (M == 1 && bgb::w1a16_decode1_supported(K))
        return finish(bgb::launch_w1a16_decode1(x, x_f16, K, N, P, alpha, a_f16, y, ydt, s));
    if (bgb::w1a16_decodem_supported(M, K))
        return finish(bgb::launch_w1a16_decodem(x, x_f16, M, K, N, P, alpha, a_f16, y, ydt, s));
    if (M <= bgb::kW1A16DecodeMaxM)
        return finish(bgb::launch_w1a16_decodek(x, x_f16, M, K, N, P, alpha, a_f16, y, ydt,
                                                static_cast<float*>(ws), s));
    return finish(bgb::launch_w1a16_gemm(static_cast<const uint16_t*>(x), x_f16, M, K, N, P, alpha, a_f16, y, ydt,
                                         lay.total ? carve(ws, lay.part) : nullptr, s));
}

int fbi_linear_w1a16(const void* x, int x_dtype, int64_t M, int64_t K, int64_t N, const uint32_t* P,
                     const void* alpha, int alpha_dtype, void* y, int y_dtype, void* ws, size_t ws_bytes,
                     void* stream) {
    bool empty = false;
    int rc = check_shape(M, K, N);
    if (rc) return rc;
    rc = fbi_dtypes(x_dtype, alpha_dtype, y_dtype);
    if (rc) return rc;
    rc = fbi_check(x, M, K, N, P, alpha, y, &empty);
    if (rc || empty) return rc;
    const size_t need = bgb::FbiLinearWs::make(M, K, N).total;
    if (need && (!ws || ws_bytes < need || !aligned16(ws))) return BGB_EINVAL;
    return fbi_run(x, x_dtype, M, K, N, P, alpha, alpha_dtype, y, y_dtype, ws, static_cast<hipStream_t>(stream));
}

// Byte ranges [a, a + na) and [b, b + nb) share a byte.
static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return na && nb && pa < pb + nb && pb < pa + na;
}

static int group_live(const bgb_w1a16_item* items, int count, bgb::W1a16Item* out) {
    int n = 0;
    for (int i = 0; i < count; ++i)
        if (items[i].N > 0) out[n++] = bgb::W1a16Item{items[i].x, items[i].P, items[i].alpha, items[i].y, items[i].K,
                                                      items[i].N};
    return n;
}

// 1: one single-token launch; 2: one few-token launch; 3: one launch of the
// grouped GEMM (17 to 64 tokens); 0: item by item.
static int group_one_launch(const bgb_w1a16_item* items, int count, int64_t M) {
    bgb::W1a16Item in[BGB_GROUP_MAX];
    const int n = group_live(items, count, in);
    if (M == 1) return bgb::w1a16_decode1_group_supported(in, n) ? 1 : 0;
    if (M > 16) return bgb::w1a16_gemm_group_supported(in, n, M) ? 3 : 0;
    return bgb::w1a16_decodem_group_supported(in, n, M) ? 2 : 0;
}

size_t bgb_group_workspace_bytes(const bgb_w1a16_item* items, int count, int64_t M) {
    if (!items || count <= 0 || count > BGB_GROUP_MAX || M <= 0) return 0;
    const int one = group_one_launch(items, count, M);
    if (one == 3) {
        bgb::W1a16Item in[BGB_GROUP_MAX];
        const int n = group_live(items, count, in);
        return bgb::w1a16_gemm_group_ws_bytes(in, n, M);
    }
    if (one) return 0;
    size_t need = 0;
    for (int i = 0; i < count; ++i) {
        const size_t n = bgb_workspace_bytes(BGB_OP_FBI_LINEAR, M, items[i].K, items[i].N);
        need = n > need ? n : need;
    }
    return need;
}

static_assert(BGB_GROUP_MAX == bgb::kGroupMax, "group size");

int fbi_linear_w1a16_group(const bgb_w1a16_item* items, int count, int64_t M, int x_dtype, int alpha_dtype,
                           int y_dtype, void* ws, size_t ws_bytes, void* stream) {
    if (count < 0 || count > BGB_GROUP_MAX || (count > 0 && !items) || M < 0) return BGB_EINVAL;
    int rc = fbi_dtypes(x_dtype, alpha_dtype, y_dtype);
    if (rc) return rc;
    bool live[BGB_GROUP_MAX] = {};
    int nlive = 0;
    for (int i = 0; i < count; ++i) {
        const bgb_w1a16_item& it = items[i];
        bool empty = false;
        rc = fbi_check(it.x, M, it.K, it.N, it.P, it.alpha, it.y, &empty);
        if (rc) return rc;
        live[i] = !empty;
        nlive += live[i];
    }
    if (nlive == 0) return BGB_OK;
    const size_t ysz = y_dtype == BGB_F32 ? 4 : 2, asz = alpha_dtype == BGB_F32 ? 4 : 2;
    for (int i = 0; i < count; ++i) {
        if (!live[i]) continue;
        const size_t ybytes = size_t(M) * size_t(items[i].N) * ysz;
        for (int k = 0; k < count; ++k) {
            if (!live[k]) continue;
            const bgb_w1a16_item& o = items[k];
            if (overlaps(items[i].y, ybytes, o.x, size_t(M) * size_t(o.K) * 2) ||
                overlaps(items[i].y, ybytes, o.P, bgb_packed_bytes(o.K, o.N)) ||
                overlaps(items[i].y, ybytes, o.alpha, size_t(o.N) * asz) ||
                (k != i && overlaps(items[i].y, ybytes, o.y, size_t(M) * size_t(o.N) * ysz)))
                return BGB_EINVAL;
        }
    }
    const size_t need = bgb_group_workspace_bytes(items, count, M);
    if (need && (!ws || ws_bytes < need || !aligned16(ws))) return BGB_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int one = group_one_launch(items, count, M);
    if (one) {
        bgb::W1a16Item in[BGB_GROUP_MAX];
        const int n = group_live(items, count, in);
        const int ydt = y_dtype == BGB_F32 ? 0 : (y_dtype == BGB_F16 ? 1 : 2);
        const int xf = x_dtype == BGB_F16, af = alpha_dtype == BGB_F16;
        if (one == 3) return finish(bgb::launch_w1a16_gemm_group(in, n, M, xf, af, ydt, ws, s));
        return finish(one == 1 ? bgb::launch_w1a16_decode1_group(in, n, xf, af, ydt, s)
                               : bgb::launch_w1a16_decodem_group(in, n, M, xf, af, ydt, s));
    }
    // Up to 16 tokens with some items too large for the one-launch form (the
    // tokens do not fit in LDS whole): the others still go as one group
    // launch when there are at least two of them, the rest one by one (the
    // items are independent, so the order does not matter).
    bool alone[BGB_GROUP_MAX] = {};
    if (M <= 16) {
        bgb::W1a16Item fit[BGB_GROUP_MAX];
        int nf = 0;
        for (int i = 0; i < count; ++i) {
            if (!live[i]) continue;
            const bool ok = M == 1 ? bgb::w1a16_decode1_group_item_ok(items[i].K)
                                   : bgb::w1a16_decodem_supported(M, items[i].K);
            if (ok)
                fit[nf++] = bgb::W1a16Item{items[i].x, items[i].P, items[i].alpha, items[i].y, items[i].K,
                                           items[i].N};
            else
                alone[i] = true;
        }
        if (nf >= 2) {
            const int ydt = y_dtype == BGB_F32 ? 0 : (y_dtype == BGB_F16 ? 1 : 2);
            const int xf = x_dtype == BGB_F16, af = alpha_dtype == BGB_F16;
            rc = finish(M == 1 ? bgb::launch_w1a16_decode1_group(fit, nf, xf, af, ydt, s)
                               : bgb::launch_w1a16_decodem_group(fit, nf, M, xf, af, ydt, s));
            if (rc) return rc;
        } else {
            for (int i = 0; i < count; ++i) alone[i] = live[i];
        }
    } else {
        for (int i = 0; i < count; ++i) alone[i] = live[i];
    }
    for (int i = 0; i < count; ++i) {
        if (!alone[i]) continue;
        const bgb_w1a16_item& it = items[i];
        rc = fbi_run(it.x, x_dtype, M, it.K, it.N, it.P, it.alpha, alpha_dtype, it.y, y_dtype, ws, s);
        if (rc) return rc;
    }
    return BGB_OK;
}

int fbi_pack_transposed(const uint32_t* P, int64_t K, int64_t N, uint32_t* PT, void* stream) {
    int rc = check_shape(0, K, N);
    if (rc) return rc;
    if (N % 32 != 0 || 2 * N > bgb::kMaxK) return BGB_EINVAL;
    if (N == 0) return BGB_OK;
    if (!P || !PT || !aligned16(P) || !aligned16(PT)) return BGB_EINVAL;
    if (overlaps(P, bgb_packed_bytes(K, N), PT, bgb_packed_bytes(2 * N, K))) return BGB_EINVAL;
    return finish(bgb::launch_pack_transpose(P, K, N, PT, static_cast<hipStream_t>(stream)));
}

int fbi_linear_w1a16_backward(const void* dy, const void* x, int dtype, int64_t M, int64_t K, int64_t N,
                              const uint32_t* P, const uint32_t* PT, const void* alpha, int alpha_dtype, void* dx,
                              int dx_dtype, float* dalpha, float* dw, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(M, K, N);
    if (rc) return rc;
    if (dtype != BGB_BF16 && dtype != BGB_F16) return BGB_EUNSUPPORTED;
    if (alpha_dtype != BGB_F32 && alpha_dtype != BGB_F16) return BGB_EUNSUPPORTED;
    if (dx && dx_dtype != BGB_F32 && dx_dtype != BGB_BF16 && dx_dtype != BGB_F16) return BGB_EUNSUPPORTED;
    if (N % 32 != 0 || 2 * N > bgb::kMaxK || M * 2 * N > kMaxElems) return BGB_EINVAL;
    // dX runs the forward product over [S^T; S^T], a 2N x K operand: it must
    // meet the forward's own shape limits too
    if (dx && N > 0 && (rc = check_shape(M, 2 * N, K))) return rc;
    if (M == 0 || N == 0) return BGB_OK;          // empty: nothing is read or written
    if (!dy || !alpha || !aligned16(dy) || !aligned16(alpha)) return BGB_EINVAL;
    if (dx && (!PT || !aligned16(PT) || !aligned16(dx))) return BGB_EINVAL;
    if ((dalpha || dw) && (!x || !aligned16(x))) return BGB_EINVAL;
    if (dalpha && (!P || !aligned16(P) || !aligned16(dalpha))) return BGB_EINVAL;
    if (dw && !aligned16(dw)) return BGB_EINVAL;
    const bgb::FbiBackwardWs lay = bgb::FbiBackwardWs::make(M, K, N);
    if (!ws || ws_bytes < lay.total || !aligned16(ws)) return BGB_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int f16 = dtype == BGB_F16, a_f16 = alpha_dtype == BGB_F16;
    uint16_t* g2 = dx ? reinterpret_cast<uint16_t*>(carve(ws, lay.g2)) : nullptr;
    float* ones = reinterpret_cast<float*>(carve(ws, lay.ones));
    void* inner = carve(ws, lay.inner);
    rc = finish(bgb::launch_fbi_backward_parts(dy, f16, x, M, K, N, alpha, a_f16, g2, ones, K > N ? K : N, dw, s));
    if (rc) return rc;
    if (dx) {                                     // dX = [g_hi g_lo] [S^T; S^T]
        rc = fbi_run(g2, BGB_BF16, M, 2 * N, K, PT, ones, BGB_F32, dx, dx_dtype, inner, s);
        if (rc) return rc;
    }
    if (dalpha) {                                 // z = x S, then dalpha = sum_m dY z
        float* z = reinterpret_cast<float*>(carve(ws, lay.z));
        rc = fbi_run(x, dtype, M, K, N, P, ones, BGB_F32, z, BGB_F32, inner, s);
        if (rc) return rc;
        double* part = reinterpret_cast<double*>(carve(ws, lay.part));
        rc = finish(bgb::launch_dalpha(dy, f16, z, M, N, part, dalpha, s));
    }
    return rc;
}

// Shared checks of the BitLinear entry points; fills qb/lim from qp.
static int bitlinear_params(const bgb_quant_params* qp, bgb_quant_params* p, float* qb, float* lim) {
    *p = bgb_quant_params{1e-5, 8, 1e-3f, BGB_ROUND_TRUNC, BGB_GAMMA_TENSOR, BGB_RANGE_SYMMETRIC};
    if (qp) *p = *qp;
    if (p->bits < 2 || p->bits > 8) return BGB_EUNSUPPORTED;
    if ((p->round_mode != BGB_ROUND_TRUNC && p->round_mode != BGB_ROUND_RNE) ||
        (p->gamma_scope != BGB_GAMMA_TENSOR && p->gamma_scope != BGB_GAMMA_TOKEN) ||
        (p->act_range != BGB_RANGE_SYMMETRIC && p->act_range != BGB_RANGE_NONNEG))
        return BGB_EUNSUPPORTED;
    if (!(p->ln_eps > 0.0) || !(p->q_eps > 0.0f) || !(p->q_eps < 1.0f)) return BGB_EINVAL;
    *qb = float(1 << (p->bits - 1));
    *lim = *qb - p->q_eps;                       // fl32(Q_b - eps), as the reference computes it
    return BGB_OK;
}

int bitlinear_quantize(const void* x, int x_dtype, int64_t M, int64_t K, const bgb_quant_params* qp,
                       int8_t* xq_opt, float* gamma_opt, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_shape(M, K, 0);
    if (rc) return rc;
    if (x_dtype != BGB_F32 && x_dtype != BGB_BF16) return BGB_EUNSUPPORTED;
    bgb_quant_params p;
    float qb, lim;
    if ((rc = bitlinear_params(qp, &p, &qb, &lim))) return rc;
    if (M == 0) return BGB_OK;                    // empty: nothing is read or written
    if (!x || !aligned16(x)) return BGB_EINVAL;
    if ((gamma_opt && (reinterpret_cast<uintptr_t>(gamma_opt) & 3u)) || (xq_opt && !aligned16(xq_opt)))
        return BGB_EINVAL;
    const bgb::BitlinearWs lay = bgb::BitlinearWs::make(M, K, 0);
    if (!ws || ws_bytes < lay.total || !aligned16(ws)) return BGB_EINVAL;
    const bool decode = M <= bgb::kGemvMaxM;
    float* mins = p.act_range == BGB_RANGE_NONNEG ? reinterpret_cast<float*>(carve(ws, lay.mins)) : nullptr;
    return finish(bgb::launch_ln_quant(x, x_dtype == BGB_BF16, M, K, p.ln_eps, qb, lim,
                                       p.round_mode == BGB_ROUND_RNE, p.gamma_scope == BGB_GAMMA_TOKEN, mins,
                                       p.q_eps, decode ? 0 : 1,
                                       reinterpret_cast<int8_t*>(carve(ws, lay.q)),
                                       reinterpret_cast<int32_t*>(carve(ws, lay.rowsum)),
                                       reinterpret_cast<float*>(carve(ws, lay.stats)),
                                       reinterpret_cast<float*>(carve(ws, lay.gamma)), xq_opt, gamma_opt,
                                       static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Product + epilogue from the codes in the workspace (binary or ternary weights).
int matmul_impl(int64_t M, int64_t K, int64_t N, const uint32_t* P, const float* beta, const bgb_quant_params* qp,
                float* y, int32_t* acc_opt, void* ws, size_t ws_bytes, void* stream, bool tern) {
    int rc = check_shape(M, K, N);
    if (rc) return rc;
    bgb_quant_params p;
    float qb, lim;
    if ((rc = bitlinear_params(qp, &p, &qb, &lim))) return rc;
    if (M == 0 || N == 0) return BGB_OK;          // empty: nothing is read or written
    if (!P || !beta || !y || !aligned16(P) || !aligned16(y)) return BGB_EINVAL;
    if (reinterpret_cast<uintptr_t>(beta) & 3u) return BGB_EINVAL;
    if (acc_opt && !aligned16(acc_opt)) return BGB_EINVAL;
    const bgb::BitlinearWs lay = bgb::BitlinearWs::make(M, K, N, tern);
    if (!ws || ws_bytes < lay.total || !aligned16(ws)) return BGB_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int8_t* q = reinterpret_cast<const int8_t*>(carve(ws, lay.q));
    const int32_t* rowsum = reinterpret_cast<const int32_t*>(carve(ws, lay.rowsum));
    // one gamma for the tensor, or each token's own: the row maxima the
    // prologue keeps in its statistics ([M][3]: mu32, rstd32, max |h|)
    const bool token = p.gamma_scope == BGB_GAMMA_TOKEN;
    const float* gamma = token ? reinterpret_cast<const float*>(carve(ws, lay.stats)) + 2
                               : reinterpret_cast<const float*>(carve(ws, lay.gamma));
    const int gstride = token ? 3 : 0;
    if (M <= bgb::kGemvMaxM)
        return finish(bgb::launch_w1a8_gemv(q, rowsum, gamma, gstride, beta, qb, M, K, N, P, y, acc_opt, tern, s));
    return finish(bgb::launch_w1a8_gemm(q, rowsum, gamma, gstride, beta, qb, M, K, N, P, y, acc_opt,
                                        carve(ws, lay.part), tern, s));
}

// Prologue + product (one fused launch for a single token).
int forward_impl(const void* x, int x_dtype, int64_t M, int64_t K, int64_t N, const uint32_t* P, const float* beta,
                 const bgb_quant_params* qp, float* y, int8_t* xq_opt, float* gamma_opt, int32_t* acc_opt, void* ws,
                 size_t ws_bytes, void* stream, bool tern) {
    int rc = check_shape(M, K, N);
    if (rc) return rc;
    if (x_dtype != BGB_F32 && x_dtype != BGB_BF16) return BGB_EUNSUPPORTED;
    bgb_quant_params p;
    float qb, lim;
    if ((rc = bitlinear_params(qp, &p, &qb, &lim))) return rc;
    if (M == 0 || N == 0) return BGB_OK;          // empty: nothing is read or written
    if (!x || !P || !beta || !y) return BGB_EINVAL;
    if (!aligned16(x) || !aligned16(P) || !aligned16(y)) return BGB_EINVAL;
    if ((reinterpret_cast<uintptr_t>(beta) & 3u) || (gamma_opt && (reinterpret_cast<uintptr_t>(gamma_opt) & 3u)))
        return BGB_EINVAL;
    if ((xq_opt && !aligned16(xq_opt)) || (acc_opt && !aligned16(acc_opt))) return BGB_EINVAL;
    const bgb::BitlinearWs lay = bgb::BitlinearWs::make(M, K, N, tern);
    if (!ws || ws_bytes < lay.total || !aligned16(ws)) return BGB_EINVAL;
    if (M == 1 && bgb::w1a8_decode1_supported(K) && p.act_range == BGB_RANGE_SYMMETRIC) {
        // one token: its gamma is the tensor's, whatever the scope (the
        // non-negative range runs the two-stage path)
        return finish(bgb::launch_w1a8_decode1(x, x_dtype == BGB_BF16, K, N, p.ln_eps, qb, lim,
                                               p.round_mode == BGB_ROUND_RNE, P, beta, y, acc_opt, xq_opt, gamma_opt,
                                               tern, static_cast<hipStream_t>(stream)));
    }
    rc = bitlinear_quantize(x, x_dtype, M, K, qp, xq_opt, gamma_opt, ws, ws_bytes, stream);
    if (rc) return rc;
    return matmul_impl(M, K, N, P, beta, qp, y, acc_opt, ws, ws_bytes, stream, tern);
}

}  // namespace

extern "C" {

int bitlinear_matmul(int64_t M, int64_t K, int64_t N, const uint32_t* P, const float* beta,
                     const bgb_quant_params* qp, float* y, int32_t* acc_opt, void* ws, size_t ws_bytes,
                     void* stream) {
    return matmul_impl(M, K, N, P, beta, qp, y, acc_opt, ws, ws_bytes, stream, false);
}

int bitlinear_w1a8(const void* x, int x_dtype, int64_t M, int64_t K, int64_t N, const uint32_t* P,
                   const float* beta, const bgb_quant_params* qp, float* y, int8_t* xq_opt, float* gamma_opt,
                   int32_t* acc_opt, void* ws, size_t ws_bytes, void* stream) {
    return forward_impl(x, x_dtype, M, K, N, P, beta, qp, y, xq_opt, gamma_opt, acc_opt, ws, ws_bytes, stream, false);
}

int bitlinear158_matmul(int64_t M, int64_t K, int64_t N, const uint32_t* P, const float* beta,
                        const bgb_quant_params* qp, float* y, int32_t* acc_opt, void* ws, size_t ws_bytes,
                        void* stream) {
    return matmul_impl(M, K, N, P, beta, qp, y, acc_opt, ws, ws_bytes, stream, true);
}

int bitlinear158_w1a8(const void* x, int x_dtype, int64_t M, int64_t K, int64_t N, const uint32_t* P,
                      const float* beta, const bgb_quant_params* qp, float* y, int8_t* xq_opt, float* gamma_opt,
                      int32_t* acc_opt, void* ws, size_t ws_bytes, void* stream) {
    return forward_impl(x, x_dtype, M, K, N, P, beta, qp, y, xq_opt, gamma_opt, acc_opt, ws, ws_bytes, stream, true);
}

const char* bgb_status_string(int status) {
    switch (status) {
        case BGB_OK: return "ok";
        case BGB_EINVAL: return "invalid argument (null pointer, shape, alignment or workspace size)";
        case BGB_EUNSUPPORTED: return "unsupported dtype or mode";
        case BGB_EHIP: return "HIP launch failed (see bgb_last_hip_error)";
        case BGB_ESCRATCH: return "the call needs more workspace than the no-alloc entry point's static scratch holds";
        default: return "unknown status";
    }
}

int bgb_last_hip_error(void) { return g_last_hip_error; }

const char* bgb_version(void) { return "bgb 0.1.0 gfx950"; }

}  // extern "C"
