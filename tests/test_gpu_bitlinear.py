"""GPU parity: bitlinear_w1a8 (LN + absmax prologue, W1A8 product, epilogue)
against the oracle: gamma and codes bit-exact, int32 accumulators bit-exact,
outputs within 1e-5 of the fp64 epilogue."""
import numpy as np
import pytest
import torch

import bgb_synth as syn
from gpu_util import check_w1a8, dev_bits16, dev_f32, host_f32, say, to_bits

pytestmark = pytest.mark.gpu


def _run(bgb, orc, W, x_host, x_dev, qp=None, bits=8):
    K, N = W.shape
    P, beta, centre = bgb.binarize_pack(dev_f32(W), bgb.MODE_BITNET)
    y, ex = bgb.bitlinear_w1a8(x_dev, P, beta, N, qp, want_q=True, want_gamma=True, want_acc=True)
    torch.cuda.synchronize()
    c_ref, b_ref = orc.bitnet_scalars(W)
    rm, gs = (qp.round_mode, qp.gamma_scope) if qp else (0, 0)
    q_ref, g_ref, _, _ = orc.ln_absmax_quant(x_host, bits=bits, round_mode=rm, gamma_scope=gs)
    g = host_f32(ex["gamma"]).astype(np.float32)
    assert np.array_equal(g.view(np.uint32), np.atleast_1d(g_ref).view(np.uint32)), (g, g_ref)
    q = ex["q"].cpu().numpy()
    assert np.array_equal(q, q_ref), f"{int((q != q_ref).sum())} codes differ"
    acc_ref = orc.bitlinear_acc(q_ref, W, c_ref)
    acc = ex["acc"].cpu().numpy().astype(np.int64)
    assert np.array_equal(acc, acc_ref)
    y_ref = orc.bitlinear_out(acc_ref, b_ref, g_ref, bits=bits)
    return to_bits(y), y_ref


CASES = [(1, 4096, 11008), (1, 96, 65), (1, 16416, 40), (3, 160, 300), (16, 768, 260), (17, 96, 65),
         # single token, 4-wave blocks (N < 8192) with up to 16 pieces per thread,
         # and 8-wave blocks at the largest fused K
         (1, 11008, 4096), (1, 16384, 300), (1, 8320, 8192), (1, 16384, 8200),
         (40, 1024, 300), (64, 512, 100), (65, 256, 90), (130, 256, 513), (5, 11008, 64),
         # GEMM pipeline: 1, 3 or 0 tail stages of the 4-stage ring, ragged M/N
         (150, 640, 300), (257, 896, 520), (300, 1024, 1000)]


@pytest.mark.parametrize("M,K,N", CASES)
@pytest.mark.parametrize("x_kind", ["f32", "bf16"])
def test_bitlinear_parity(bgb_gpu, orc, M, K, N, x_kind):
    say(f"bitlinear M={M} K={K} N={N} x={x_kind}")
    seed = 500 + M + K
    W = syn.normal_f32(seed, 0, (K, N), mean=0.001, std=0.02)
    xf = syn.normal_f32(seed, 1, (M, K))
    if x_kind == "bf16":
        xb = syn.f32_to_bf16_bits(xf)
        x_host = syn.bf16_bits_to_f32(xb)
        x_dev = dev_bits16(xb, torch.bfloat16)
    else:
        x_host, x_dev = xf, dev_f32(xf)
    y, y_ref = _run(bgb_gpu, orc, W, x_host, x_dev)
    check_w1a8(y, y_ref, f"M={M} K={K} N={N}")


def test_bitlinear_quant_closed_forms(bgb_gpu, orc):
    """Rows (-3,-1,1,3)... give codes (-127,-42,42,127); constant rows give 0."""
    say("bitlinear closed forms")
    K, N = 96, 40
    x = np.tile(np.array([-3, -1, 1, 3], np.float32), (4, K // 4))
    x[2] = 0.75
    W = syn.normal_f32(3, 0, (K, N), mean=0.001, std=0.02)
    y, y_ref = _run(bgb_gpu, orc, W, x, dev_f32(x))
    check_w1a8(y, y_ref)


@pytest.mark.parametrize("bits", [4, 8])
def test_bitlinear_bits_and_all_tie_weights(bgb_gpu, orc, bits):
    """Constant W: every weight ties to -1, so acc = -sum(q) for every column."""
    say(f"bitlinear constant weights bits={bits}")
    from bit_gemm_binarize_amd import QuantParams
    K, N = 256, 33
    W = np.full((K, N), 0.37, np.float32)
    for M in (2, 20):
        xf = syn.normal_f32(4, 1, (M, K))
        y, y_ref = _run(bgb_gpu, orc, W, xf, dev_f32(xf), qp=QuantParams(bits=bits), bits=bits)
        check_w1a8(y, y_ref)


def test_bitlinear_zero_input(bgb_gpu, orc):
    say("bitlinear zero input")
    K, N = 128, 20
    W = syn.normal_f32(5, 0, (K, N), mean=0.001, std=0.02)
    for M in (1, 18):
        x = np.zeros((M, K), np.float32)
        y, y_ref = _run(bgb_gpu, orc, W, x, dev_f32(x))
        assert np.all(y == 0) and np.all(y_ref == 0)


def test_bitlinear_empty_and_deterministic(bgb_gpu):
    say("bitlinear empty + determinism")
    K, N = 1024, 300
    P, beta, _ = bgb_gpu.binarize_pack(dev_f32(syn.normal_f32(6, 0, (K, N), mean=0.001, std=0.02)),
                                       bgb_gpu.MODE_BITNET)
    assert bgb_gpu.bitlinear_w1a8(torch.zeros((0, K), device="cuda"), P, beta, N).shape == (0, N)
    for M in (1, 70):
        x = dev_f32(syn.normal_f32(6, 1, (M, K)))
        ys = [bgb_gpu.bitlinear_w1a8(x, P, beta, N) for _ in range(5)]
        torch.cuda.synchronize()
        for t in ys[1:]:
            assert torch.equal(ys[0], t)


@pytest.mark.parametrize("M,K,N", [(1, 4096, 11008), (1, 768, 300), (9, 768, 300), (40, 512, 200), (70, 512, 200)])
def test_stage_api_matches_single_call(bgb_gpu, M, K, N):
    """bitlinear_quantize + bitlinear_matmul (two launches) and bitlinear_w1a8
    (fused into one launch for a single token) give bit-identical results,
    and one quantization serves several weights."""
    say(f"bitlinear stage API M={M} K={K} N={N}")
    x = dev_f32(syn.normal_f32(600 + M, 1, (M, K)))
    Ws = [syn.normal_f32(600 + M, 10 + i, (K, N), mean=0.001, std=0.02) for i in range(2)]
    packs = [bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_BITNET) for W in Ws]
    ws = torch.empty(bgb_gpu.workspace_bytes(bgb_gpu.OP_BITLINEAR, M, K, N), dtype=torch.uint8, device="cuda")
    taps = bgb_gpu.bitlinear_quantize(x, ws=ws, want_q=True, want_gamma=True)
    outs = [bgb_gpu.bitlinear_matmul(M, K, P, beta, N, ws=ws, want_acc=True) for P, beta, _ in packs]
    for (P, beta, _), (y2, acc2) in zip(packs, outs):
        y1, ex = bgb_gpu.bitlinear_w1a8(x, P, beta, N, want_q=True, want_gamma=True, want_acc=True)
        torch.cuda.synchronize()
        assert torch.equal(ex["q"], taps["q"])
        assert torch.equal(ex["gamma"], taps["gamma"])
        assert torch.equal(ex["acc"], acc2)
        assert torch.equal(y1, y2)


OPT_CASES = [(1, 4096, 11008), (1, 16416, 40), (5, 768, 260), (16, 1024, 300), (17, 512, 65), (40, 1024, 300),
             (150, 640, 300)]


@pytest.mark.parametrize("M,K,N", OPT_CASES)
@pytest.mark.parametrize("rm,gs", [(1, 0), (0, 1), (1, 1)])
def test_bitlinear_quantizer_options(bgb_gpu, orc, M, K, N, rm, gs):
    """Round-to-nearest codes and per-token gamma through every prologue and
    product path (fused single token, one-block prologue + GEMV, two-pass
    prologue + GEMV, GEMM): gamma(s) and codes bit-exact, acc exact, y to 1e-5
    of the fp64 epilogue with each token's own gamma."""
    from bit_gemm_binarize_amd import QuantParams
    say(f"bitlinear options round={rm} scope={gs} M={M} K={K} N={N}")
    seed = 700 + M + K
    W = syn.normal_f32(seed, 0, (K, N), mean=0.001, std=0.02)
    xf = syn.normal_f32(seed, 1, (M, K))
    xf[:, ::7] *= np.float32(1.5)                     # heavier tails, token maxima spread out
    y, y_ref = _run(bgb_gpu, orc, W, xf, dev_f32(xf), qp=QuantParams(round_mode=rm, gamma_scope=gs))
    check_w1a8(y, y_ref, f"round={rm} scope={gs} M={M} K={K} N={N}")


@pytest.mark.parametrize("M", [2, 40])
def test_bitlinear_option_closed_forms(bgb_gpu, orc, M):
    """Hand-derived codes: rows (-3,-1,1,3) round to (-127,-43,43,127);
    rows (-0.7,0.7) beside them give +-95 with one gamma and +-127 with
    their own."""
    from bit_gemm_binarize_amd import QuantParams
    say(f"bitlinear option closed forms M={M}")
    K, N = 96, 40
    x = np.empty((M, K), np.float32)
    x[0::2] = np.tile(np.array([-3, -1, 1, 3], np.float32), K // 4)
    x[1::2] = np.tile(np.array([-0.7, 0.7], np.float32), K // 2)
    W = syn.normal_f32(8, 0, (K, N), mean=0.001, std=0.02)
    P, beta, _ = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_BITNET)
    expect = {(1, 0): ([-127, -43, 43, 127], [-95, 95]), (0, 1): ([-127, -42, 42, 127], [-127, 127]),
              (1, 1): ([-127, -43, 43, 127], [-127, 127])}
    for (rm, gs), (e0, e1) in expect.items():
        _, ex = bgb_gpu.bitlinear_w1a8(dev_f32(x), P, beta, N, QuantParams(round_mode=rm, gamma_scope=gs),
                                       want_q=True)
        q = ex["q"].cpu().numpy()
        assert np.array_equal(q[0::2], np.tile(np.array(e0, np.int8), (q[0::2].shape[0], K // 4))), (rm, gs)
        assert np.array_equal(q[1::2], np.tile(np.array(e1, np.int8), (q[1::2].shape[0], K // 2))), (rm, gs)


@pytest.mark.parametrize("M,K,N", [(1, 768, 300), (9, 768, 300), (40, 512, 200)])
def test_stage_api_token_scope(bgb_gpu, M, K, N):
    """The two-stage API with per-token gamma and rounding matches the single call."""
    from bit_gemm_binarize_amd import QuantParams
    say(f"bitlinear stage API options M={M}")
    qp = QuantParams(round_mode=1, gamma_scope=1)
    x = dev_f32(syn.normal_f32(650 + M, 1, (M, K)))
    P, beta, _ = bgb_gpu.binarize_pack(dev_f32(syn.normal_f32(650 + M, 2, (K, N), mean=0.001, std=0.02)),
                                       bgb_gpu.MODE_BITNET)
    ws = torch.empty(bgb_gpu.workspace_bytes(bgb_gpu.OP_BITLINEAR, M, K, N), dtype=torch.uint8, device="cuda")
    taps = bgb_gpu.bitlinear_quantize(x, qp, ws=ws, want_q=True, want_gamma=True)
    y2, acc2 = bgb_gpu.bitlinear_matmul(M, K, P, beta, N, qp, ws=ws, want_acc=True)
    y1, ex = bgb_gpu.bitlinear_w1a8(x, P, beta, N, qp, want_q=True, want_gamma=True, want_acc=True)
    torch.cuda.synchronize()
    assert taps["gamma"].shape == (M,) and torch.equal(ex["gamma"], taps["gamma"])
    assert torch.equal(ex["q"], taps["q"]) and torch.equal(ex["acc"], acc2) and torch.equal(y1, y2)


@pytest.mark.parametrize("kind", ["n01", "shift3", "shift1000", "near_const"])
@pytest.mark.parametrize("K", [96, 4096, 16384])
@pytest.mark.parametrize("x_kind", ["f32", "bf16"])
def test_bitlinear_single_token_statistics_paths(bgb_gpu, orc, kind, K, x_kind):
    """One token through the fused kernel. Its LayerNorm statistics take one
    fp64 pass (sum x, sum x^2) and fall back to the two-pass variance when the
    one-pass value could round differently in fp32: rows with a mean far from
    zero (N(1000, 1)) always take the fallback (the one-pass error bound spans
    several fp32 values there), nearly constant rows sit where the bound is a
    fraction of an fp32 ulp, N(0, 1) and N(3, 0.5) rows take the single pass.
    gamma, codes and acc must be bit-exact."""
    say(f"bitlinear single token statistics {kind} K={K} x={x_kind}")
    N = 200
    seed = 1500 + K
    W = syn.normal_f32(seed, 0, (K, N), mean=0.001, std=0.02)
    xf = syn.normal_f32(seed, 1 + len(kind), (1, K))
    if kind == "shift3":
        xf = xf * np.float32(0.5) + np.float32(3.0)
    elif kind == "shift1000":
        xf = xf + np.float32(1000.0)
    elif kind == "near_const":
        xf = np.full((1, K), np.float32(0.37), np.float32)
        xf[0, K // 3] = np.float32(0.375)
    xf = np.ascontiguousarray(xf, np.float32)
    if x_kind == "bf16":
        xb = syn.f32_to_bf16_bits(xf)
        x_host, x_dev = syn.bf16_bits_to_f32(xb), dev_bits16(xb, torch.bfloat16)
    else:
        x_host, x_dev = xf, dev_f32(xf)
    y, y_ref = _run(bgb_gpu, orc, W, x_host, x_dev)
    check_w1a8(y, y_ref, f"{kind} K={K}")
