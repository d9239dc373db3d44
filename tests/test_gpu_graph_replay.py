"""HIP-graph replays of the library calls: every replay must reproduce the
eager result bit for bit, with eager work and synchronizations in between
(the benchmark times graph replays)."""
import numpy as np
import pytest
import torch

import bgb_synth as syn
from gpu_util import dev_bits16, dev_f32, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K", [(1, 1024), (16, 1024), (40, 1024), (24, 8192)])   # the last: K split
def test_graph_replays_match_eager(bgb_gpu, M, K):
    say(f"graph replay M={M} K={K}")
    N = 700
    W = dev_f32(syn.normal_f32(31, 0, (K, N), mean=0.001, std=0.02))
    Pf, alpha = bgb_gpu.binarize_pack(W, bgb_gpu.MODE_FBI)
    Pb, beta, _ = bgb_gpu.binarize_pack(W, bgb_gpu.MODE_BITNET)
    xf = dev_f32(syn.normal_f32(31, 1, (M, K)))
    xb = dev_bits16(syn.f32_to_bf16_bits(syn.normal_f32(31, 2, (M, K))), torch.bfloat16)
    ref16 = bgb_gpu.fbi_linear_w1a16(xb, Pf, alpha, N, torch.bfloat16)
    ref8 = bgb_gpu.bitlinear_w1a8(xf, Pb, beta, N)
    y16 = torch.empty_like(ref16)
    y8 = torch.empty_like(ref8)
    ws16 = torch.empty(max(bgb_gpu.workspace_bytes(bgb_gpu.OP_FBI_LINEAR, M, K, N), 256), dtype=torch.uint8,
                       device="cuda")
    ws8 = torch.empty(bgb_gpu.workspace_bytes(bgb_gpu.OP_BITLINEAR, M, K, N), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bgb_gpu.fbi_linear_w1a16(xb, Pf, alpha, N, y=y16, ws=ws16)
        bgb_gpu.bitlinear_w1a8(xf, Pb, beta, N, y=y8, ws=ws8)
    for rep in range(4):
        y16.zero_()
        y8.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y16, ref16), rep
        assert torch.equal(y8, ref8), rep
        # eager work between replays, reusing the same workspaces
        bgb_gpu.bitlinear_w1a8(xf * 2, Pb, beta, N, ws=ws8)
        torch.cuda.synchronize()


@pytest.mark.parametrize("M", [1, 4, 40])
def test_graph_replays_group_and_backward(bgb_gpu, M):
    """The group call (one launch at 1 and 4 tokens; at 40 the grouped GEMM
    and its reduce pass over the parts' sums in the workspace) and the FBI
    backward (split gradient, forward kernels, token sums, dW) replayed from
    a graph: bit for bit equal to the eager calls on every replay."""
    say(f"graph replay group + backward M={M}")
    shapes = [(1024, 512), (2048, 256), (512, 1024)]
    lin, Ps = [], []
    for i, (K, N) in enumerate(shapes):
        W = dev_f32(syn.normal_f32(41 + i, 0, (K, N), std=0.02))
        P, a = bgb_gpu.binarize_pack(W, bgb_gpu.MODE_FBI, torch.float16)
        x = dev_bits16(syn.f32_to_bf16_bits(syn.normal_f32(41 + i, 1, (M, K))), torch.bfloat16)
        lin.append((x, P, a, N))
        Ps.append(P)
    ref = bgb_gpu.fbi_linear_w1a16_group(lin, torch.bfloat16)
    ys = [torch.empty_like(r) for r in ref]
    K, N = shapes[0]
    x0, P0, a0, _ = lin[0]
    PT = bgb_gpu.fbi_pack_transposed(P0, K, N)
    dy = dev_bits16(syn.f32_to_bf16_bits(syn.normal_f32(49, 2, (M, N))), torch.bfloat16)
    rdx, rda, rdw = bgb_gpu.fbi_linear_w1a16_backward(dy, x0, P0, PT, a0)
    wsg = torch.empty(max(bgb_gpu.group_workspace_bytes([(x, P, a, y) for (x, P, a, _), y in zip(lin, ys)], M),
                          256), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(bgb_gpu.workspace_bytes(bgb_gpu.OP_FBI_BACKWARD, M, K, N), dtype=torch.uint8, device="cuda")
    dx = torch.empty_like(rdx)
    da = torch.empty(max(N, 4), dtype=torch.float32, device="cuda")[:N]
    dw = torch.empty_like(rdw)
    lib = bgb_gpu.load()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bgb_gpu.fbi_linear_w1a16_group(lin, ys=ys, ws=wsg)
        rc = lib.fbi_linear_w1a16_backward(dy.data_ptr(), x0.data_ptr(), 2, M, K, N, P0.data_ptr(), PT.data_ptr(),
                                           a0.data_ptr(), 1, dx.data_ptr(), 0, da.data_ptr(), dw.data_ptr(),
                                           wsb.data_ptr(), wsb.numel(), torch.cuda.current_stream().cuda_stream)
        assert rc == 0
    for rep in range(3):
        for y in ys:
            y.zero_()
        dx.zero_()
        da.zero_()
        dw.zero_()
        g.replay()
        torch.cuda.synchronize()
        for y, r in zip(ys, ref):
            assert torch.equal(y, r), rep
        assert torch.equal(dx, rdx) and torch.equal(da, rda) and torch.equal(dw, rdw), rep
        bgb_gpu.fbi_linear_w1a16_backward(dy, x0, P0, PT, a0, ws=wsb)      # eager work on the same workspace
        torch.cuda.synchronize()
