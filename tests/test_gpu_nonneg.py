"""GPU parity: the non-negative activation range (BitNet blog, section 一,
eq. (6)) through every prologue and product path, against the oracle: gamma
and codes bit-exact, int32 accumulators bit-exact, outputs within 1e-5 of the
fp64 epilogue of eq. (7)."""
import numpy as np
import pytest
import torch

import bgb_synth as syn
from conftest import read_golden
from gpu_util import check_w1a8, dev_bits16, dev_f32, host_f32, say, to_bits

pytestmark = pytest.mark.gpu


def _run(bgb, orc, W, x_host, x_dev, rm, gs, bits=8, tern=False):
    from bit_gemm_binarize_amd import QuantParams, RANGE_NONNEG
    K, N = W.shape
    qp = QuantParams(bits=bits, round_mode=rm, gamma_scope=gs, act_range=RANGE_NONNEG)
    if tern:
        P, beta, _ = bgb.binarize_pack(dev_f32(W), bgb.MODE_TERNARY)
        y, ex = bgb.bitlinear158_w1a8(x_dev, P, beta, N, qp, want_q=True, want_gamma=True, want_acc=True)
    else:
        P, beta, _ = bgb.binarize_pack(dev_f32(W), bgb.MODE_BITNET)
        y, ex = bgb.bitlinear_w1a8(x_dev, P, beta, N, qp, want_q=True, want_gamma=True, want_acc=True)
    torch.cuda.synchronize()
    q_ref, g_ref, _ = orc.ln_nonneg_quant(x_host, bits=bits, round_mode=rm, gamma_scope=gs)
    g = host_f32(ex["gamma"]).astype(np.float32)
    assert np.array_equal(g.view(np.uint32), np.atleast_1d(g_ref).view(np.uint32)), (g, g_ref)
    q = ex["q"].cpu().numpy()
    assert np.array_equal(q, q_ref), f"{int((q != q_ref).sum())} codes differ"
    assert q.min() >= 0
    if tern:
        T, gw = orc.ternary(W)
        acc_ref = orc.int8_acc(q_ref, T)
        b_ref = gw
    else:
        c_ref, b_ref = orc.bitnet_scalars(W)
        acc_ref = orc.bitlinear_acc(q_ref, W, c_ref)
    acc = ex["acc"].cpu().numpy().astype(np.int64)
    assert np.array_equal(acc, acc_ref)
    y_ref = orc.bitlinear_out(acc_ref, b_ref, g_ref, bits=bits)
    return to_bits(y), y_ref


CASES = [(1, 4096, 11008), (1, 96, 65), (3, 160, 300), (16, 768, 260), (17, 96, 65), (40, 1024, 300),
         (64, 512, 100), (65, 256, 90), (150, 640, 300)]


@pytest.mark.parametrize("M,K,N", CASES)
@pytest.mark.parametrize("rm,gs", [(0, 0), (1, 1)])
def test_nonneg_parity(bgb_gpu, orc, M, K, N, rm, gs):
    say(f"nonneg range M={M} K={K} N={N} round={rm} scope={gs}")
    seed = 900 + M + K
    W = syn.normal_f32(seed, 0, (K, N), mean=0.001, std=0.02)
    xf = syn.normal_f32(seed, 1, (M, K))
    xf[:, ::5] *= np.float32(2.0)                     # skewed rows: the minimum differs from -max |h|
    y, y_ref = _run(bgb_gpu, orc, W, xf, dev_f32(xf), rm, gs)
    check_w1a8(y, y_ref, f"nonneg M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", [(1, 1024, 300), (20, 512, 130), (100, 256, 96)])
def test_nonneg_bf16_and_ternary(bgb_gpu, orc, M, K, N):
    say(f"nonneg range bf16 / ternary M={M} K={K} N={N}")
    seed = 950 + M
    W = syn.normal_f32(seed, 0, (K, N), mean=0.001, std=0.02)
    xb = syn.f32_to_bf16_bits(syn.normal_f32(seed, 1, (M, K)))
    x_host = syn.bf16_bits_to_f32(xb)
    for tern in (False, True):
        y, y_ref = _run(bgb_gpu, orc, W, x_host, dev_bits16(xb, torch.bfloat16), 0, 0, tern=tern)
        check_w1a8(y, y_ref, f"nonneg tern={tern} M={M}")


@pytest.mark.parametrize("M", [1, 2, 40])
def test_nonneg_golden_closed_forms(bgb_gpu, orc, M):
    """Hand-derived codes of eq. (6) (tests/golden/quant_nonneg_closed_forms.txt)."""
    from bit_gemm_binarize_amd import QuantParams, RANGE_NONNEG
    say(f"nonneg golden M={M}")
    g = read_golden("quant_nonneg_closed_forms.txt")
    K, N = 128, 48
    W = syn.normal_f32(7, 0, (K, N), mean=0.001, std=0.02)
    P, beta, _ = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_BITNET)
    for pat, qk, bits, rm in [("pattern_a", "nn_q_a", 8, 0), ("pattern_d", "nn4_rne_q_d", 4, 1),
                              ("pattern_d", "nn4_q_d", 4, 0)]:
        period = np.array([float(v) for v in g[pat]], np.float32)
        expect = np.array([int(v) for v in g[qk]], np.int8)
        x = np.tile(period, (M, K // period.size))
        qp = QuantParams(bits=bits, round_mode=rm, act_range=RANGE_NONNEG)
        _, ex = bgb_gpu.bitlinear_w1a8(dev_f32(x), P, beta, N, qp, want_q=True)
        torch.cuda.synchronize()
        assert np.array_equal(ex["q"].cpu().numpy(), np.tile(expect, (M, K // period.size))), (pat, qk, M)
