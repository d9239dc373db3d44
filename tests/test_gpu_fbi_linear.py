"""GPU parity: fbi_linear_w1a16 (decode kernels for M <= 64, MFMA GEMM above)
against the fp64 oracle, plus exactness probes that pin the bit layout."""
import numpy as np
import pytest
import torch

import bgb_synth as syn
from gpu_util import check_w1a16, dev_bits16, dev_f32, say, to_bits

pytestmark = pytest.mark.gpu

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _x_bits(x_kind, seed, M, K, scale=1.0):
    a = syn.normal_f32(seed, 1, (M, K)) * np.float32(scale)
    return syn.f32_to_bf16_bits(a) if x_kind == "bf16" else syn.f32_to_f16_bits(a)


def _run(bgb, orc, W, xb, x_kind, y_kind, adt="f32"):
    K, N = W.shape
    P, alpha = bgb.binarize_pack(dev_f32(W), bgb.MODE_FBI, TORCH_DT[adt])
    x = dev_bits16(xb, TORCH_DT[x_kind])
    y = bgb.fbi_linear_w1a16(x, P, alpha, N, TORCH_DT[y_kind])
    torch.cuda.synchronize()
    a_host = alpha.detach().float().cpu().numpy().astype(np.float32)
    ref = orc.fbi_linear(xb, W, a_host, x_kind)
    return to_bits(y), ref, a_host


CASES = [
    # (M, K, N) covering every dispatch path: single-token fused decode (M = 1,
    # K <= 16384), single token beyond the fused size (K staged in chunks),
    # 2..16 tokens staged whole in LDS, 2..64 tokens staged in chunks, and the
    # MFMA GEMM (M > 64, split-K plans for small M x N); ragged N and K tails.
    (1, 768, 768), (1, 11008, 100), (1, 16416, 40), (8, 768, 768), (3, 96, 65), (16, 160, 300),
    (1, 16384, 4000), (1, 16384, 8200), (1, 11008, 4096),
    # 2..16 tokens staged in LDS by every block (one group per block, two,
    # K split over 1..8 waves), and sizes just past what fits (two launches)
    (2, 16384, 300), (4, 11008, 4096), (5, 11008, 100), (6, 11008, 70), (12, 2048, 1000), (16, 4096, 4100),
    (16, 4096, 12288), (2, 1024, 40000),
    # two tokens whose K fits in LDS but needs more than 8 steps per wave:
    # the chunked kernel takes them
    (2, 33024, 40),
    # 2..64 tokens with K staged in chunks: 16 or 32 tokens per block, one or
    # more token blocks, chunk tails, K beyond the fused single-token size, K
    # split over 3..17 blocks per column block (raw sums, then the reduce pass)
    (16, 11008, 4096), (24, 1024, 520), (33, 5632, 300), (64, 2048, 6144), (48, 352, 100), (20, 16416, 70),
    (5, 4096, 33), (17, 96, 65), (40, 768, 260), (64, 2048, 520), (65, 256, 300), (130, 256, 300),
    (200, 352, 513),
    # GEMM pipeline: 4-stage ring with 0 or 2 tail stages, ragged M/N, padded K
    (150, 640, 300), (257, 1024, 1000), (300, 4000, 257),
]


@pytest.mark.parametrize("M,K,N", CASES)
@pytest.mark.parametrize("y_kind", ["f32", "bf16"])
def test_fbi_linear_bf16_parity(bgb_gpu, orc, M, K, N, y_kind):
    say(f"fbi_linear bf16 M={M} K={K} N={N} y={y_kind}")
    W = syn.normal_f32(100 + M + K, 0, (K, N), std=0.02)
    xb = _x_bits("bf16", 100 + M + K, M, K)
    y, ref, _ = _run(bgb_gpu, orc, W, xb, "bf16", y_kind)
    check_w1a16(y, ref, y_kind, f"M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", [(1, 768, 768), (7, 160, 300), (16, 4096, 64), (40, 768, 260), (64, 96, 65),
                                   (24, 11008, 200), (129, 96, 65)])
@pytest.mark.parametrize("y_kind", ["f32", "f16"])
def test_fbi_linear_f16_parity(bgb_gpu, orc, M, K, N, y_kind):
    say(f"fbi_linear f16 M={M} K={K} N={N} y={y_kind}")
    W = syn.normal_f32(200 + M, 0, (K, N), std=0.02)
    xb = _x_bits("f16", 200 + M, M, K)
    y, ref, _ = _run(bgb_gpu, orc, W, xb, "f16", y_kind, adt="f16")
    check_w1a16(y, ref, y_kind, f"f16 M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N", [(1, 96, 65), (1, 4096, 300), (5, 1024, 300), (16, 4096, 70), (40, 1024, 300),
                                   (64, 512, 33), (20, 16416, 70), (131, 96, 257)])
@pytest.mark.parametrize("x_kind", ["bf16", "f16"])
def test_fbi_linear_integer_activations_bit_exact(bgb_gpu, orc, M, K, N, x_kind):
    """Integer-valued activations (|x| <= 16) make every partial sum exact in
    fp32 whatever the order, so the fp32 output must equal fl32(alpha * S)."""
    say(f"fbi_linear integer-exact {x_kind} M={M} K={K} N={N}")
    rng = syn.rng_for(300 + M, 2)
    xf = rng.integers(-16, 17, size=(M, K)).astype(np.float32)
    xb = syn.f32_to_bf16_bits(xf) if x_kind == "bf16" else syn.f32_to_f16_bits(xf)
    W = syn.normal_f32(300 + M, 0, (K, N), std=0.02)
    y, ref, _ = _run(bgb_gpu, orc, W, xb, x_kind, "f32")
    assert np.array_equal(y.astype(np.float32), ref.astype(np.float32))


@pytest.mark.parametrize("K,N", [(96, 65), (768, 300), (4096, 20)])
def test_unit_vector_probes_read_back_signs(bgb_gpu, orc, K, N):
    """x = e_k gives y_j = alpha_j s_kj exactly: reads row k of the signs through
    the kernel, pinning bit order and layout without trusting P."""
    say(f"fbi_linear unit probes K={K} N={N}")
    W = syn.normal_f32(400 + K, 0, (K, N), std=0.02)
    ks = sorted(set([0, 1, 15, 16, 17, 31, 32, 63, 64, 100 % K, K - 33, K - 1]))
    for M in (1, len(ks[:16]), 40, 100):
        rows = (ks * (M // len(ks) + 1))[:M]
        e = np.zeros((M, K), np.float32)
        e[np.arange(M), rows] = 1.0
        y, ref, a = _run(bgb_gpu, orc, W, syn.f32_to_bf16_bits(e), "bf16", "f32")
        S = orc.sign_fbi(W)
        assert np.array_equal(y.astype(np.float32), (a[None, :] * S[rows].astype(np.float32)))


def test_fbi_linear_trained_alpha_and_closed_forms(bgb_gpu, orc):
    """All-positive weights give y = alpha * sum(x); a caller-supplied alpha is used as is."""
    say("fbi_linear closed forms")
    K, N = 256, 48
    for M in (3, 33):
        xb = _x_bits("bf16", 7, M, K)
        xf = syn.bf16_bits_to_f32(xb).astype(np.float64)
        W = np.full((K, N), 0.5, np.float32)
        P, alpha = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_FBI)
        custom = np.linspace(-2, 3, N).astype(np.float32)
        y = bgb_gpu.fbi_linear_w1a16(dev_bits16(xb, torch.bfloat16), P, dev_f32(custom), N)
        torch.cuda.synchronize()
        ref = xf.sum(1)[:, None] * custom[None, :].astype(np.float64)
        check_w1a16(to_bits(y), ref, "f32", "closed form")


def test_fbi_linear_empty_and_deterministic(bgb_gpu):
    say("fbi_linear empty + determinism")
    K, N = 1024, 300
    W = dev_f32(syn.normal_f32(9, 0, (K, N), std=0.02))
    P, alpha = bgb_gpu.binarize_pack(W, bgb_gpu.MODE_FBI)
    x0 = torch.zeros((0, K), dtype=torch.bfloat16, device="cuda")
    assert bgb_gpu.fbi_linear_w1a16(x0, P, alpha, N).shape == (0, N)
    for M in (4, 64):
        x = dev_bits16(_x_bits("bf16", 9, M, K), torch.bfloat16)
        ys = [bgb_gpu.fbi_linear_w1a16(x, P, alpha, N) for _ in range(5)]
        torch.cuda.synchronize()
        for t in ys[1:]:
            assert torch.equal(ys[0], t)


@pytest.mark.parametrize("K,N", [(4096, 4096), (11008, 700), (768, 768), (96, 65)])
@pytest.mark.parametrize("x_kind", ["bf16", "f16"])
def test_single_token_wide_range_bound(bgb_gpu, orc, K, N, x_kind):
    """One token: the activations' exponents spread over many binades. The
    single-token kernels carry the token, scaled by a power of two so that its
    largest magnitude lies in [8, 16), as five limbs of quantum 2^-16, so each
    activation is off by at most max|x| 2^-20; every limb column sums exactly
    on the matrix cores, and the final fp32 combine and the alpha product round
    a few times. So |y_j - ref_j| <= |alpha_j| (K max|x| 2^-20 + sum|x| 2^-20),
    beside the 2e-3 normwise tolerance."""
    say(f"single token wide range K={K} N={N} x={x_kind}")
    W = syn.normal_f32(700 + K, 0, (K, N), std=0.02)
    spread = 6.0 if x_kind == "bf16" else 2.0          # f16 keeps its values inside its range
    a = syn.normal_f32(701, 1, (1, K)) * np.exp2(np.round(syn.normal_f32(701, 2, (1, K)) * spread))
    xb = syn.f32_to_bf16_bits(a.astype(np.float32)) if x_kind == "bf16" else syn.f32_to_f16_bits(a.astype(np.float32))
    y, ref, a_host = _run(bgb_gpu, orc, W, xb, x_kind, "f32")
    xv = (syn.bf16_bits_to_f32(xb) if x_kind == "bf16" else syn.f16_bits_to_f32(xb)).astype(np.float64)
    xm, xs = np.abs(xv).max(), np.abs(xv).sum()
    bound = np.abs(a_host.astype(np.float64)) * (K * xm + xs) * 2.0 ** -20
    assert np.all(np.abs(y[0] - ref[0]) <= bound), float(np.max(np.abs(y[0] - ref[0]) / bound))
    check_w1a16(y, ref, "f32", "wide range")


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
def test_single_token_non_finite_gives_nan(bgb_gpu, orc, bad):
    """A token holding an inf or a NaN: every output of the single-token kernels is NaN."""
    say(f"single token non-finite {bad}")
    K, N = 1024, 300
    W = syn.normal_f32(710, 0, (K, N), std=0.02)
    a = syn.normal_f32(711, 1, (1, K))
    a[0, 17] = bad
    xb = syn.f32_to_bf16_bits(a.astype(np.float32))
    P, alpha = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_FBI)
    y = bgb_gpu.fbi_linear_w1a16(dev_bits16(xb, torch.bfloat16), P, alpha, N)
    torch.cuda.synchronize()
    assert np.all(np.isnan(to_bits(y)))
