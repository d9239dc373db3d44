"""GPU parity at the five workloads' own shapes, seeds and dtypes.

Full outputs are compared where the oracle finishes in seconds; at prefill
sizes a fixed set of rows (tile edges plus seeded random rows) is compared
against the oracle run on exactly those rows, which computes each output
independently of the others.
"""
import numpy as np
import pytest
import torch

import bgb_synth as syn
from gpu_util import check_w1a16, check_w1a8, dev_bits16, dev_f32, host_bits16, host_f32, host_u32, say, to_bits

pytestmark = pytest.mark.gpu


def sample_rows(M, seed, n_random=12):
    edges = {0, 1, 15, 16, 63, 64, 127, 128, M // 2, M - 129, M - 128, M - 2, M - 1}
    rnd = syn.rng_for(seed, 77).choice(M, size=n_random, replace=False)
    return np.array(sorted({int(r) for r in edges | set(rnd.tolist()) if 0 <= r < M}))


def test_fbi_768_config(bgb_gpu, orc):
    c = syn.CONFIGS["fbi_768"]
    say("config fbi_768")
    W = syn.normal_f32(c["seed"], 0, (c["K"], c["N"]), std=c["w_std"])
    xb = syn.f32_to_bf16_bits(syn.normal_f32(c["seed"], 1, (c["M"], c["K"])))
    P, alpha = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_FBI)
    y = bgb_gpu.fbi_linear_w1a16(dev_bits16(xb, torch.bfloat16), P, alpha, c["N"])
    torch.cuda.synchronize()
    a_ref = orc.fbi_alpha(W)
    assert np.array_equal(host_u32(P), orc.pack(orc.sign_fbi(W)))
    assert np.array_equal(host_f32(alpha), a_ref)
    check_w1a16(to_bits(y), orc.fbi_linear(xb, W, a_ref), "f32", "fbi_768")


@pytest.mark.parametrize("stages", [False, True])
def test_bitlinear_decode_config(bgb_gpu, orc, stages):
    c = syn.CONFIGS["bitlinear_decode_4096x11008"]
    say(f"config bitlinear decode stages={stages}")
    K, N, M = c["K"], c["N"], c["M"]
    W = syn.normal_f32(c["seed"], 0, (K, N), mean=c["w_mean"], std=c["w_std"])
    x = syn.normal_f32(c["seed"], 1, (M, K))
    P, beta, centre = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_BITNET)
    if stages:
        ws = torch.empty(bgb_gpu.workspace_bytes(bgb_gpu.OP_BITLINEAR, M, K, N), dtype=torch.uint8, device="cuda")
        taps = bgb_gpu.bitlinear_quantize(dev_f32(x), ws=ws, want_q=True, want_gamma=True)
        y, acc = bgb_gpu.bitlinear_matmul(M, K, P, beta, N, ws=ws, want_acc=True)
        q, g = taps["q"], taps["gamma"]
    else:
        y, ex = bgb_gpu.bitlinear_w1a8(dev_f32(x), P, beta, N, want_q=True, want_gamma=True, want_acc=True)
        q, g, acc = ex["q"], ex["gamma"], ex["acc"]
    torch.cuda.synchronize()
    c_ref, b_ref = orc.bitnet_scalars(W)
    assert host_f32(centre)[0] == c_ref and host_f32(beta)[0] == b_ref
    assert np.array_equal(host_u32(P), orc.pack(orc.sign_bitnet(W, c_ref)))
    q_ref, g_ref, _, _ = orc.ln_absmax_quant(x)
    assert np.float32(host_f32(g)[0]) == g_ref
    assert np.array_equal(q.cpu().numpy(), q_ref)
    acc_ref = orc.bitlinear_acc(q_ref, W, c_ref)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
    check_w1a8(to_bits(y), orc.bitlinear_out(acc_ref, b_ref, g_ref), "bitlinear decode")


@pytest.mark.parametrize("B", [1, 4, 16])
def test_w1a16_decode_7b_layer_config(bgb_gpu, orc, B):
    c = syn.CONFIGS["w1a16_decode_7b_layer"]
    say(f"config 7B layer decode B={B}")
    done = set()
    for li, (name, K, N) in enumerate(c["shapes"]):
        if (K, N) in done:       # q/k/v/o share a shape; gate/up share one
            continue
        done.add((K, N))
        W = syn.normal_f32(c["seed"], li, (K, N), std=c["w_std"])
        xb = syn.f32_to_bf16_bits(syn.normal_f32(c["seed"], 100 + li, (B, K)))
        P, alpha = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_FBI, torch.float16)
        y = bgb_gpu.fbi_linear_w1a16(dev_bits16(xb, torch.bfloat16), P, alpha, N, torch.bfloat16)
        torch.cuda.synchronize()
        a16 = orc.f32_to_f16(orc.fbi_alpha(W))
        assert np.array_equal(host_bits16(alpha), a16)
        check_w1a16(to_bits(y), orc.fbi_linear(xb, W, orc.f16_to_f32(a16)), "bf16", f"7B {name} B={B}")


def test_w1a16_prefill_config(bgb_gpu, orc):
    c = syn.CONFIGS["w1_prefill_4096x4096x11008"]
    say("config prefill W1A16 4096x4096x11008")
    M, K, N = c["M"], c["K"], c["N"]
    W = syn.normal_f32(c["seed"], 0, (K, N), std=c["w_std"])
    xb = syn.f32_to_bf16_bits(syn.normal_f32(c["seed"], 1, (M, K)))
    P, alpha = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_FBI)
    y = bgb_gpu.fbi_linear_w1a16(dev_bits16(xb, torch.bfloat16), P, alpha, N, torch.bfloat16)
    torch.cuda.synchronize()
    a_ref = orc.fbi_alpha(W)
    assert np.array_equal(host_f32(alpha), a_ref)
    rows = sample_rows(M, c["seed"])
    ref = orc.fbi_linear(np.ascontiguousarray(xb[rows]), W, a_ref)
    check_w1a16(to_bits(y)[rows], ref, "bf16", "prefill W1A16")


def test_w1a8_prefill_config(bgb_gpu, orc):
    c = syn.CONFIGS["w1_prefill_4096x4096x11008"]
    say("config prefill W1A8 4096x4096x11008")
    M, K, N = c["M"], c["K"], c["N"]
    W = syn.normal_f32(c["seed"], 0, (K, N), std=c["w_std"])
    xb = syn.f32_to_bf16_bits(syn.normal_f32(c["seed"], 1, (M, K)))
    P, beta, _ = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_BITNET)
    y, ex = bgb_gpu.bitlinear_w1a8(dev_bits16(xb, torch.bfloat16), P, beta, N, want_q=True, want_gamma=True,
                                   want_acc=True)
    torch.cuda.synchronize()
    c_ref, b_ref = orc.bitnet_scalars(W)
    q_ref, g_ref, _, _ = orc.ln_absmax_quant(syn.bf16_bits_to_f32(xb))
    assert np.float32(host_f32(ex["gamma"])[0]) == g_ref
    assert np.array_equal(ex["q"].cpu().numpy(), q_ref)           # every code of the 4096 x 4096 tensor
    rows = sample_rows(M, c["seed"])
    acc_ref = orc.bitlinear_acc(np.ascontiguousarray(q_ref[rows]), W, c_ref)
    assert np.array_equal(ex["acc"].cpu().numpy()[rows].astype(np.int64), acc_ref)
    check_w1a8(to_bits(y)[rows], orc.bitlinear_out(acc_ref, b_ref, g_ref), "prefill W1A8")


@pytest.mark.parametrize("phase", ["decode_b64", "prefill_2x1024"])
def test_1p3b_stack_config(bgb_gpu, orc, phase):
    c = syn.CONFIGS["w1a16_1p3b_stack"]
    M = c["decode_batch"] if phase == "decode_b64" else c["prefill_tokens"]
    say(f"config 1.3B stack {phase} M={M}")
    done = set()
    for li, (name, K, N) in enumerate(c["shapes"]):
        if (K, N) in done:
            continue
        done.add((K, N))
        W = syn.normal_f32(c["seed"], li, (K, N), std=c["w_std"])
        xb = syn.f32_to_bf16_bits(syn.normal_f32(c["seed"], 100 + li, (M, K)))
        P, alpha = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_FBI, torch.float16)
        y = bgb_gpu.fbi_linear_w1a16(dev_bits16(xb, torch.bfloat16), P, alpha, N, torch.bfloat16)
        torch.cuda.synchronize()
        a16 = orc.f32_to_f16(orc.fbi_alpha(W))                     # the stored f16 scale
        assert np.array_equal(host_bits16(alpha), a16)
        rows = np.arange(M) if M <= 64 else sample_rows(M, c["seed"], 8)
        ref = orc.fbi_linear(np.ascontiguousarray(xb[rows]), W, orc.f16_to_f32(a16))
        check_w1a16(to_bits(y)[rows], ref, "bf16", f"1.3B {name} {phase}")
