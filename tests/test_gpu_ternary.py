"""GPU parity: BitNet b1.58 ternary weights ("BitNet b1.58: 1bit LLM时代",
section 二, eq. (9)-(11)) -- the two-plane pack bit-exact with gamma_w, and
the W1.58A8 forward (same activation prologue as BitLinear) with codes and
int32 accumulators bit-exact and outputs within 1e-5 of the fp64 epilogue."""
import numpy as np
import pytest
import torch

import bgb_synth as syn
from gpu_util import check_w1a8, dev_bits16, dev_f32, host_f32, say, to_bits

pytestmark = pytest.mark.gpu

EPS_W = 1e-5   # the library's eps in RoundClip(W / (gamma_w + eps), -1, 1)


def _pack(bgb, orc, W):
    K, N = W.shape
    P2, beta, _ = bgb.binarize_pack(dev_f32(W), bgb.MODE_TERNARY)
    torch.cuda.synchronize()
    T, g = orc.ternary(W, eps_w=EPS_W)
    words = P2.cpu().numpy().view(np.uint32)[:2 * orc.packed_words(K, N)]
    assert np.array_equal(words, orc.pack_ternary(T)), "ternary planes differ"
    b = np.float32(host_f32(beta)[0])
    assert b.view(np.uint32) == g.view(np.uint32), (b, g)
    return P2, beta, T, g


@pytest.mark.parametrize("K,N", [(96, 65), (160, 300), (4096, 1000), (11008, 64), (32, 1)])
def test_ternary_pack_parity(bgb_gpu, orc, K, N):
    say(f"ternary pack K={K} N={N}")
    W = syn.normal_f32(800 + K, 0, (K, N), mean=0.001, std=0.02)
    W[0, 0] = 0.0
    _pack(bgb_gpu, orc, W)


def _forward(bgb, orc, W, x_host, x_dev, qp=None):
    K, N = W.shape
    P2, beta, T, g_w = _pack(bgb, orc, W)
    y, ex = bgb.bitlinear158_w1a8(x_dev, P2, beta, N, qp, want_q=True, want_gamma=True, want_acc=True)
    torch.cuda.synchronize()
    rm, gs = (qp.round_mode, qp.gamma_scope) if qp else (0, 0)
    q_ref, g_ref, _, _ = orc.ln_absmax_quant(x_host, round_mode=rm, gamma_scope=gs)
    g = host_f32(ex["gamma"]).astype(np.float32)
    assert np.array_equal(g.view(np.uint32), np.atleast_1d(g_ref).view(np.uint32))
    assert np.array_equal(ex["q"].cpu().numpy(), q_ref)
    acc_ref = orc.int8_acc(q_ref, T)
    assert np.array_equal(ex["acc"].cpu().numpy().astype(np.int64), acc_ref)
    return to_bits(y), orc.bitlinear_out(acc_ref, g_w, g_ref)


CASES = [(1, 4096, 11008), (1, 96, 65), (1, 11008, 4096), (1, 16384, 300), (3, 160, 300), (16, 768, 260),
         (17, 96, 65), (32, 1024, 300), (40, 1024, 300), (65, 256, 90), (150, 640, 300), (257, 896, 520)]


@pytest.mark.parametrize("M,K,N", CASES)
@pytest.mark.parametrize("x_kind", ["f32", "bf16"])
def test_ternary_forward_parity(bgb_gpu, orc, M, K, N, x_kind):
    say(f"ternary forward M={M} K={K} N={N} x={x_kind}")
    seed = 900 + M + K
    W = syn.normal_f32(seed, 0, (K, N), mean=0.001, std=0.02)
    xf = syn.normal_f32(seed, 1, (M, K))
    if x_kind == "bf16":
        xb = syn.f32_to_bf16_bits(xf)
        x_host, x_dev = syn.bf16_bits_to_f32(xb), dev_bits16(xb, torch.bfloat16)
    else:
        x_host, x_dev = xf, dev_f32(xf)
    y, y_ref = _forward(bgb_gpu, orc, W, x_host, x_dev)
    check_w1a8(y, y_ref, f"ternary M={M} K={K} N={N}")


@pytest.mark.parametrize("M", [1, 20, 70])
def test_ternary_closed_form(bgb_gpu, orc, M):
    """W = c * pattern: the planes read back the pattern, and acc = sum pattern q."""
    say(f"ternary closed form M={M}")
    rng = syn.rng_for(44, M)
    K, N = 256, 37
    pat = rng.integers(-1, 2, size=(K, N)).astype(np.int8)
    pat[0] = 1
    W = pat.astype(np.float32) * np.float32(0.05)
    xf = syn.normal_f32(45, M, (M, K))
    P2, beta, T, _ = _pack(bgb_gpu, orc, W)
    assert np.array_equal(T, pat)
    _, ex = bgb_gpu.bitlinear158_w1a8(dev_f32(xf), P2, beta, N, want_q=True, want_acc=True)
    q = ex["q"].cpu().numpy().astype(np.int64)
    assert np.array_equal(ex["acc"].cpu().numpy().astype(np.int64), q @ pat.astype(np.int64))


@pytest.mark.parametrize("M,K,N", [(1, 768, 300), (9, 768, 300), (40, 512, 200)])
@pytest.mark.parametrize("rm,gs", [(0, 0), (1, 1)])
def test_ternary_stage_api_and_options(bgb_gpu, orc, M, K, N, rm, gs):
    """bitlinear_quantize + bitlinear158_matmul equal the single call, also
    with round-to-nearest codes and per-token gamma; both match the oracle."""
    from bit_gemm_binarize_amd import QuantParams
    say(f"ternary stage API M={M} round={rm} scope={gs}")
    qp = QuantParams(round_mode=rm, gamma_scope=gs)
    W = syn.normal_f32(950 + M, 0, (K, N), mean=0.001, std=0.02)
    xf = syn.normal_f32(950 + M, 1, (M, K))
    y, y_ref = _forward(bgb_gpu, orc, W, xf, dev_f32(xf), qp)
    check_w1a8(y, y_ref)
    P2, beta, _ = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_TERNARY)
    x = dev_f32(xf)
    ws = torch.empty(bgb_gpu.workspace_bytes(bgb_gpu.OP_BITLINEAR158, M, K, N), dtype=torch.uint8, device="cuda")
    bgb_gpu.bitlinear_quantize(x, qp, ws=ws)
    y2, acc2 = bgb_gpu.bitlinear158_matmul(M, K, P2, beta, N, qp, ws=ws, want_acc=True)
    y1, ex = bgb_gpu.bitlinear158_w1a8(x, P2, beta, N, qp, want_acc=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(ex["acc"], acc2)


def test_ternary_deterministic(bgb_gpu):
    say("ternary determinism")
    K, N = 1024, 300
    W = dev_f32(syn.normal_f32(46, 0, (K, N), mean=0.001, std=0.02))
    P2, beta, _ = bgb_gpu.binarize_pack(W, bgb_gpu.MODE_TERNARY)
    for M in (1, 20, 100):
        x = dev_f32(syn.normal_f32(46, M, (M, K)))
        ys = [bgb_gpu.bitlinear158_w1a8(x, P2, beta, N) for _ in range(4)]
        torch.cuda.synchronize()
        for t in ys[1:]:
            assert torch.equal(ys[0], t)
