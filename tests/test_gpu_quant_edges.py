"""GPU parity of the BitLinear quantizer on its edge inputs ("BitNet b1.58:
1bit LLM时代" blog, section 一, eq. (4)-(6)):

* rows whose quotients h Q_b / gamma are exact integers or half-integers, the
  only inputs that decide a code exactly at a boundary (and so force the
  exact division behind the kernels' fast reciprocal path);
* activations at subnormal scale, where gamma < Q_b / FLT_MAX and Q_b / gamma
  overflows fp32.

Each runs through every prologue path (one token: the fused decode kernel,
or the two-stage path for the non-negative range; 2 tokens: the one-block
prologue; 40 tokens: the statistics + quantization kernels and the MFMA
product), f32 and bf16 activations, truncation and rounding, both ranges.
gamma, codes and int32 accumulators must equal the oracle's bit for bit, and
the codes the hand-derived ones in tests/golden/."""
import numpy as np
import pytest
import torch

import bgb_synth as syn
from conftest import read_golden
from gpu_util import check_w1a8, dev_bits16, dev_f32, host_f32, say, to_bits

pytestmark = pytest.mark.gpu

N = 300


def _inputs(kind: str, M: int):
    """(x float32 [M][K], expected codes [M][K] for (range, round)) from the golden files."""
    g = read_golden("quant_closed_forms.txt")
    gn = read_golden("quant_nonneg_closed_forms.txt")
    if kind == "subnormal":
        e, K = int(g["subnormal_exponent"][0]), int(g["subnormal_K"][0])
        x = np.zeros((M, K), np.float32)
        hot = (37 * np.arange(M)) % K
        x[np.arange(M), hot] = np.float32(2.0 ** e)
        sym = np.zeros((M, K), np.int8)
        sym[np.arange(M), hot] = int(g["subnormal_q0"][0])
        nn = np.zeros((M, K), np.int8)
        nn[np.arange(M), hot] = int(gn["nn_subnormal_q0"][0])
        return x, {("sym", 0): sym, ("sym", 1): sym, ("nonneg", 0): nn, ("nonneg", 1): nn}
    pat, keys = {"exact_int": ("pattern_e", ("q_e", "rne_q_e")),
                 "half_int": ("pattern_f", ("q_f", "rne_q_f"))}[kind]
    period = np.array([float(v) for v in g[pat]], np.float32)
    K = 1024
    reps = K // period.size
    x = np.tile(period, (M, reps))
    exp = {("sym", rm): np.tile(np.array([int(v) for v in g[k]], np.int8), (M, reps)) for rm, k in enumerate(keys)}
    if kind == "exact_int":
        nn = np.tile(np.array([int(v) for v in gn["nn_q_e"]], np.int8), (M, reps))
        exp[("nonneg", 0)] = exp[("nonneg", 1)] = nn
    return x, exp


@pytest.mark.parametrize("kind", ["subnormal", "exact_int", "half_int"])
@pytest.mark.parametrize("M", [1, 2, 40])
@pytest.mark.parametrize("x_kind", ["f32", "bf16"])
@pytest.mark.parametrize("rng", ["sym", "nonneg"])
@pytest.mark.parametrize("rm", [0, 1])
def test_quant_edge_inputs(bgb_gpu, orc, kind, M, x_kind, rng, rm):
    from bit_gemm_binarize_amd import QuantParams, RANGE_NONNEG, RANGE_SYMMETRIC
    x, expect = _inputs(kind, M)
    if (rng, rm) not in expect:
        pytest.skip("no hand-derived codes for this range on this pattern")
    say(f"quant edges kind={kind} M={M} x={x_kind} range={rng} round={rm}")
    K = x.shape[1]
    if x_kind == "bf16":
        xb = syn.f32_to_bf16_bits(x)
        x_host = syn.bf16_bits_to_f32(xb)
        assert np.array_equal(x_host, x)            # every value is exact in bf16
        x_dev = dev_bits16(xb, torch.bfloat16)
    else:
        x_host, x_dev = x, dev_f32(x)
    W = syn.normal_f32(1200 + M + K, 0, (K, N), mean=0.001, std=0.02)
    qp = QuantParams(round_mode=rm, act_range=RANGE_NONNEG if rng == "nonneg" else RANGE_SYMMETRIC)
    P, beta, _ = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_BITNET)
    y, ex = bgb_gpu.bitlinear_w1a8(x_dev, P, beta, N, qp, want_q=True, want_gamma=True, want_acc=True)
    torch.cuda.synchronize()
    if rng == "nonneg":
        q_ref, g_ref, _ = orc.ln_nonneg_quant(x_host, round_mode=rm)
    else:
        q_ref, g_ref, _, _ = orc.ln_absmax_quant(x_host, round_mode=rm)
    assert np.array_equal(q_ref, expect[(rng, rm)])           # the oracle meets the hand derivation
    g = host_f32(ex["gamma"]).astype(np.float32)
    assert np.array_equal(g.view(np.uint32), np.atleast_1d(g_ref).view(np.uint32)), (g, g_ref)
    q = ex["q"].cpu().numpy()
    assert np.array_equal(q, q_ref), f"{int((q != q_ref).sum())} codes differ"
    c_ref, b_ref = orc.bitnet_scalars(W)
    acc_ref = orc.bitlinear_acc(q_ref, W, c_ref)
    assert np.array_equal(ex["acc"].cpu().numpy().astype(np.int64), acc_ref)
    check_w1a8(to_bits(y), orc.bitlinear_out(acc_ref, b_ref, g_ref), f"{kind} M={M}", acc=acc_ref)


@pytest.mark.parametrize("kind", ["subnormal", "exact_int"])
def test_quant_edge_inputs_ternary_single_token(bgb_gpu, orc, kind):
    """The fused single-token kernel's ternary variant shares the code path."""
    say(f"quant edges ternary kind={kind}")
    x, expect = _inputs(kind, 1)
    K = x.shape[1]
    W = syn.normal_f32(1300 + K, 0, (K, N), std=0.02)
    P, beta, _ = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_TERNARY)
    y, ex = bgb_gpu.bitlinear158_w1a8(dev_f32(x), P, beta, N, want_q=True, want_gamma=True, want_acc=True)
    torch.cuda.synchronize()
    q_ref, g_ref, _, _ = orc.ln_absmax_quant(x)
    assert np.array_equal(q_ref, expect[("sym", 0)])
    assert np.array_equal(ex["q"].cpu().numpy(), q_ref)
    T, gw = orc.ternary(W)
    acc_ref = orc.int8_acc(q_ref, T)
    assert np.array_equal(ex["acc"].cpu().numpy().astype(np.int64), acc_ref)
    check_w1a8(to_bits(y), orc.bitlinear_out(acc_ref, gw, g_ref), f"ternary {kind}", acc=acc_ref)
