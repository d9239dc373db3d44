"""bitlinear_w1a8_noalloc (the entry point for callers that cannot allocate)
against bitlinear_w1a8 through the C ABI: the same codes, gamma, int32
accumulators and outputs bit for bit on two calls in a row, the second
smaller than the first, over the single-token, few-token and GEMM paths; the
too-large call is rejected. Both entry points run the same kernels, so the
results must agree exactly; the oracle checks the accumulators as well."""
import numpy as np
import pytest
import torch

import bgb_synth as syn
from gpu_util import dev_f32, say

pytestmark = pytest.mark.gpu


def _pair(bgb, orc, M, K, N, seed, x_kind="f32"):
    W = syn.normal_f32(seed, 0, (K, N), mean=0.001, std=0.02)
    xf = syn.normal_f32(seed, 1, (M, K))
    P, beta, _ = bgb.binarize_pack(dev_f32(W), bgb.MODE_BITNET)
    x = dev_f32(xf) if x_kind == "f32" else dev_f32(xf).to(torch.bfloat16)
    y_ref, ex = bgb.bitlinear_w1a8(x, P, beta, N, want_q=True, want_gamma=True, want_acc=True)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    q = torch.zeros((M, K), dtype=torch.int8, device="cuda")
    g = torch.zeros(1, dtype=torch.float32, device="cuda")
    acc = torch.zeros((M, N), dtype=torch.int32, device="cuda")
    bgb.bitlinear_w1a8_noalloc(x, P, beta, N, y=y, q=q, gamma=g, acc=acc)
    torch.cuda.synchronize()
    assert torch.equal(q, ex["q"]) and torch.equal(g, ex["gamma"][:1])
    assert torch.equal(acc, ex["acc"])
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))      # bit for bit
    c_ref, _ = orc.bitnet_scalars(W)
    xh = xf if x_kind == "f32" else x.float().cpu().numpy()
    q_ref, _, _, _ = orc.ln_absmax_quant(xh)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), orc.bitlinear_acc(q_ref, W, c_ref))


@pytest.mark.parametrize("first,second", [((300, 1024, 520), (1, 4096, 700)),
                                          ((40, 2048, 300), (3, 512, 100)),
                                          ((1, 11008, 4096), (1, 512, 64))])
def test_noalloc_matches_bitlinear_w1a8_twice(bgb_gpu, orc, first, second):
    for i, (M, K, N) in enumerate((first, second)):
        say(f"noalloc call {i}: M={M} K={K} N={N}")
        _pair(bgb_gpu, orc, M, K, N, 1400 + 7 * i + M, "bf16" if i else "f32")


def test_noalloc_rejects_calls_beyond_its_scratch(bgb_gpu):
    say("noalloc rejection")
    M, K, N = 8192, 8192, 64                       # 64 MiB of codes alone
    assert bgb_gpu.workspace_bytes(bgb_gpu.OP_BITLINEAR, M, K, N) > bgb_gpu.noalloc_scratch_bytes()
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    P = torch.zeros(bgb_gpu.packed_bytes(K, N) // 4, dtype=torch.int32, device="cuda")
    beta = torch.ones(1, device="cuda")
    y = torch.full((M, N), 7.0, device="cuda")
    with pytest.raises(bgb_gpu.BgbError) as e:
        bgb_gpu.bitlinear_w1a8_noalloc(x, P, beta, N, y=y)
    assert e.value.status == bgb_gpu.ESCRATCH
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())                  # nothing was written
