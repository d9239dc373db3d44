"""GPU parity: the FBI-linear backward (identity straight-through estimator)
against the fp64 oracle: the transposed sign pack bit-exact, dX / dalpha / dW
within the W1A16 tolerances, and bit-exact where every partial sum is exact."""
import numpy as np
import pytest
import torch

import bgb_synth as syn
from gpu_util import W1A16_NORMWISE_TOL, check_w1a16, dev_bits16, dev_f32, host_bits16, say, to_bits

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def _bits(kind, a):
    return syn.f32_to_bf16_bits(a) if kind == "bf16" else syn.f32_to_f16_bits(a)


def _case(bgb, seed, M, K, N, kind="bf16", adt=torch.float32, int_vals=False):
    W = syn.normal_f32(seed, 0, (K, N), std=0.02)
    if int_vals:
        rng = syn.rng_for(seed, 3)
        xf = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
        gf = rng.integers(-8, 9, size=(M, N)).astype(np.float32)
    else:
        xf = syn.normal_f32(seed, 1, (M, K))
        gf = syn.normal_f32(seed, 2, (M, N))
    xb, gb = _bits(kind, xf), _bits(kind, gf)
    P, alpha = bgb.binarize_pack(dev_f32(W), bgb.MODE_FBI, adt)
    PT = bgb.fbi_pack_transposed(P, K, N)
    return W, xb, gb, P, PT, alpha


def _normwise(got, ref, tag):
    err = np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300)
    assert err <= W1A16_NORMWISE_TOL, f"{tag} normwise err {err:.3e}"


@pytest.mark.parametrize("K,N", [(32, 32), (96, 64), (256, 96), (4096, 160), (160, 4096 + 32)])
def test_pack_transposed_bit_exact(bgb_gpu, orc, K, N):
    say(f"pack_transposed K={K} N={N}")
    W = syn.normal_f32(40 + K, 0, (K, N), std=0.02)
    P, _ = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_FBI)
    PT = bgb_gpu.fbi_pack_transposed(P, K, N)
    torch.cuda.synchronize()
    S = orc.sign_fbi(W)
    want = orc.pack(np.concatenate([S.T, S.T], axis=0))
    got = PT.cpu().numpy().view(np.uint32)[:want.size]
    assert np.array_equal(got, want)


CASES = [(1, 256, 64), (3, 96, 32), (4, 512, 96), (16, 1024, 320), (40, 768, 256), (64, 512, 160),
         (70, 512, 160), (130, 1024, 512), (257, 256, 96), (1, 4096, 11008)]


@pytest.mark.parametrize("M,K,N", CASES)
def test_backward_parity(bgb_gpu, orc, M, K, N):
    say(f"fbi backward M={M} K={K} N={N}")
    W, xb, gb, P, PT, alpha = _case(bgb_gpu, 50 + M + K, M, K, N)
    dx, da, dw = bgb_gpu.fbi_linear_w1a16_backward(dev_bits16(gb, torch.bfloat16), dev_bits16(xb, torch.bfloat16),
                                                   P, PT, alpha)
    torch.cuda.synchronize()
    a_host = alpha.detach().float().cpu().numpy().astype(np.float32)
    rdx, rda, rdw = orc.fbi_backward(xb, gb, W, a_host)
    check_w1a16(to_bits(dx), rdx, "f32", f"dX M={M} K={K} N={N}")
    _normwise(to_bits(da), rda, f"dalpha M={M} K={K} N={N}")
    check_w1a16(to_bits(dw), rdw, "f32", f"dW M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", [(2, 128, 64), (33, 256, 96), (100, 512, 128)])
@pytest.mark.parametrize("kind", ["bf16", "f16"])
def test_backward_integer_inputs_bit_exact(bgb_gpu, orc, M, K, N, kind):
    """Integer inputs (|v| <= 8) and alpha = 0.5 keep g = alpha dY, every product
    and every partial sum exact in fp32, so each output is the correctly
    rounded fp32 of the exact value."""
    say(f"fbi backward integer-exact {kind} M={M} K={K} N={N}")
    W, xb, gb, P, PT, _ = _case(bgb_gpu, 60 + M, M, K, N, kind, int_vals=True)
    alpha = torch.full((N,), 0.5, dtype=torch.float32, device="cuda")
    dx, da, dw = bgb_gpu.fbi_linear_w1a16_backward(dev_bits16(gb, TORCH_DT[kind]), dev_bits16(xb, TORCH_DT[kind]),
                                                   P, PT, alpha)
    torch.cuda.synchronize()
    rdx, rda, rdw = orc.fbi_backward(xb, gb, W, np.full(N, 0.5, np.float32), kind)
    assert np.array_equal(dx.cpu().numpy(), rdx.astype(np.float32))
    assert np.array_equal(da.cpu().numpy(), rda.astype(np.float32))
    assert np.array_equal(dw.cpu().numpy(), rdw.astype(np.float32))


def test_backward_options_and_outputs_subset(bgb_gpu, orc):
    """f16 alpha, a 16-bit dX, and only some outputs requested."""
    M, K, N = 12, 384, 128
    say("fbi backward options")
    W, xb, gb, P, PT, alpha = _case(bgb_gpu, 70, M, K, N, adt=torch.float16)
    dy, x = dev_bits16(gb, torch.bfloat16), dev_bits16(xb, torch.bfloat16)
    a_host = alpha.detach().float().cpu().numpy().astype(np.float32)
    rdx, rda, rdw = orc.fbi_backward(xb, gb, W, a_host)
    dx, da, dw = bgb_gpu.fbi_linear_w1a16_backward(dy, x, P, PT, alpha, want=("dx",), dx_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert da is None and dw is None
    check_w1a16(to_bits(dx), rdx, "bf16", "dX bf16")
    dx, da, dw = bgb_gpu.fbi_linear_w1a16_backward(dy, x, P, PT, alpha, want=("dalpha", "dw"))
    torch.cuda.synchronize()
    assert dx is None
    _normwise(to_bits(da), rda, "dalpha")
    check_w1a16(to_bits(dw), rdw, "f32", "dW")


def test_backward_deterministic(bgb_gpu):
    say("fbi backward determinism")
    M, K, N = 40, 1024, 256
    W, xb, gb, P, PT, alpha = _case(bgb_gpu, 80, M, K, N)
    dy, x = dev_bits16(gb, torch.bfloat16), dev_bits16(xb, torch.bfloat16)
    runs = [bgb_gpu.fbi_linear_w1a16_backward(dy, x, P, PT, alpha) for _ in range(3)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)


def test_backward_prefill_size_sampled(bgb_gpu, orc):
    """The benchmark's backward shape (4096 tokens, 4096 x 11008, the GEMM paths
    of dX and z, the 256-tile dW) against the oracle on samples: dX on 8 rows
    (tile edges and seeded rows), dalpha and dW on 24 columns (each computed by
    the oracle from those columns alone)."""
    M, K, N = 4096, 4096, 11008
    say(f"fbi backward sampled M={M} K={K} N={N}")
    W, xb, gb, P, PT, alpha = _case(bgb_gpu, 77, M, K, N)
    dx, da, dw = bgb_gpu.fbi_linear_w1a16_backward(dev_bits16(gb, torch.bfloat16), dev_bits16(xb, torch.bfloat16),
                                                   P, PT, alpha)
    torch.cuda.synchronize()
    a_host = alpha.detach().float().cpu().numpy().astype(np.float32)
    rng = syn.rng_for(77, 9)
    rows = np.unique(np.concatenate([[0, 127, 128, 255, M - 1], rng.choice(M, 3, replace=False)]))
    rdx, _, _ = orc.fbi_backward(xb[rows], gb[rows], W, a_host)
    check_w1a16(to_bits(dx)[rows], rdx, "f32", "dX sampled rows")
    cols = np.unique(np.concatenate([[0, 255, 256, N - 1], rng.choice(N, 20, replace=False)]))
    _, rda, rdw = orc.fbi_backward(xb, np.ascontiguousarray(gb[:, cols]), np.ascontiguousarray(W[:, cols]),
                                   a_host[cols])
    _normwise(to_bits(da)[cols], rda, "dalpha sampled columns")
    got = dw[:, torch.from_numpy(cols).cuda()].cpu().numpy().astype(np.float64)
    check_w1a16(got, rdw, "f32", "dW sampled columns")
