"""GPU parity: binarize_pack against the oracle (bit-exact words and scales)."""
import numpy as np
import pytest
import torch

import bgb_synth as syn
from gpu_util import dev_f32, host_bits16, host_f32, host_u32, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K,N,seed", [(768, 768, 0), (32, 1, 5), (96, 65, 6), (160, 300, 7), (4096, 37, 8),
                                      (11008, 260, 9)])
@pytest.mark.parametrize("adt", ["f32", "f16"])
def test_pack_fbi_bit_exact(bgb_gpu, orc, K, N, seed, adt):
    say(f"pack fbi K={K} N={N} seed={seed} alpha={adt}")
    W = syn.normal_f32(seed, 0, (K, N), std=0.02)
    P, alpha = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_FBI,
                                     torch.float16 if adt == "f16" else torch.float32)
    torch.cuda.synchronize()
    P_ref = orc.pack(orc.sign_fbi(W))
    assert np.array_equal(host_u32(P)[:P_ref.size], P_ref)
    a_ref = orc.fbi_alpha(W)
    if adt == "f32":
        assert np.array_equal(host_f32(alpha).view(np.uint32), a_ref.view(np.uint32))
    else:
        assert np.array_equal(host_bits16(alpha), orc.f32_to_f16(a_ref))


def test_pack_fbi_special_values(bgb_gpu, orc):
    say("pack fbi special values")
    tiny = np.ldexp(1.0, -149)
    vals = np.array([0.0, -0.0, tiny, -tiny, np.inf, -np.inf, np.nan, 1e-38, -1e-38, 3.0], np.float32)
    W = np.tile(vals, (96, 7))[:, :67].copy()   # every row repeats the pattern across columns
    W[5, :] = -W[5, :]
    P, alpha = bgb_gpu.binarize_pack(dev_f32(np.nan_to_num(W, nan=0.0, posinf=1.0, neginf=-1.0)), bgb_gpu.MODE_FBI)
    P2, _ = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_FBI)
    torch.cuda.synchronize()
    assert np.array_equal(host_u32(P2), orc.pack(orc.sign_fbi(W)))
    Wc = np.nan_to_num(W, nan=0.0, posinf=1.0, neginf=-1.0)
    assert np.array_equal(host_u32(P), orc.pack(orc.sign_fbi(Wc)))
    assert np.array_equal(host_f32(alpha), orc.fbi_alpha(Wc))


@pytest.mark.parametrize("K,N,seed,mean", [(4096, 11008, 1, 0.001), (96, 65, 3, 0.0), (160, 300, 4, -0.01),
                                           (32, 3, 5, 0.02)])
def test_pack_bitnet_bit_exact(bgb_gpu, orc, K, N, seed, mean):
    say(f"pack bitnet K={K} N={N} seed={seed}")
    W = syn.normal_f32(seed, 0, (K, N), mean=mean, std=0.02)
    P, beta, centre = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_BITNET)
    torch.cuda.synchronize()
    c_ref, b_ref = orc.bitnet_scalars(W)
    c = np.float32(host_f32(centre)[0])
    b = np.float32(host_f32(beta)[0])
    assert c.view(np.uint32) == c_ref.view(np.uint32), (c, c_ref)
    assert b.view(np.uint32) == b_ref.view(np.uint32), (b, b_ref)
    assert np.array_equal(host_u32(P), orc.pack(orc.sign_bitnet(W, c_ref)))


def test_pack_bitnet_ties_at_centre(bgb_gpu, orc):
    """W = 0.25 + 0.125 p, pattern summing to 0: c = 0.25 exactly and p == 0 ties to -1."""
    say("pack bitnet exact-centre ties")
    K, N = 96, 10
    i = np.arange(K)[:, None]
    p = np.where(i % 3 == 0, 0.0, np.where(i % 3 == 1, 1.0, -1.0)) * np.where(np.arange(N) % 2 == 0, 1, -1)
    W = (0.25 + 0.125 * p).astype(np.float32)
    P, beta, centre = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_BITNET)
    torch.cuda.synchronize()
    assert host_f32(centre)[0] == np.float32(0.25)
    assert np.array_equal(host_u32(P), orc.pack(orc.sign_bitnet(W, np.float32(0.25))))


def test_pack_is_deterministic(bgb_gpu):
    say("pack determinism")
    W = dev_f32(syn.normal_f32(11, 0, (4096, 1000), mean=0.001, std=0.02))
    outs = [bgb_gpu.binarize_pack(W, bgb_gpu.MODE_BITNET) for _ in range(3)]
    outs += [bgb_gpu.binarize_pack(W, bgb_gpu.MODE_FBI) for _ in range(3)]
    torch.cuda.synchronize()
    for k in range(1, 3):
        for a, b in zip(outs[0], outs[k]):
            assert torch.equal(a, b)
        for a, b in zip(outs[3], outs[3 + k]):
            assert torch.equal(a, b)
