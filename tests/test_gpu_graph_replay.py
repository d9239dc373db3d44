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
