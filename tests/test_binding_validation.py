"""The Python binding rejects arguments the kernels cannot take before any
pointer reaches the C ABI (host only: nothing here launches a kernel). The
checks run in the order dtype, shape, size, contiguity, device, so that each
is reachable with host tensors."""
import pytest
import torch

import bit_gemm_binarize_amd as bgb


@pytest.fixture(scope="module", autouse=True)
def _lib():
    bgb.load()


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def test_host_tensors_are_rejected():
    x = bf16(2, 64)
    P = torch.zeros(bgb.packed_bytes(64, 8) // 4, dtype=torch.int32)
    alpha = torch.zeros(8)
    with pytest.raises(ValueError, match="CUDA"):
        bgb.fbi_linear_w1a16(x, P, alpha, 8, y=torch.zeros(2, 8))
    with pytest.raises(ValueError, match="CUDA"):
        bgb.binarize_pack(torch.zeros(64, 8))
    with pytest.raises(ValueError, match="CUDA"):
        bgb.bitlinear_w1a8(torch.zeros(1, 64), P, torch.zeros(1), 8, y=torch.zeros(1, 8))


def test_pack_requires_float32_2d():
    with pytest.raises(ValueError, match="dtype"):
        bgb.binarize_pack(bf16(64, 8))
    with pytest.raises(ValueError, match="2-D"):
        bgb.binarize_pack(torch.zeros(64))


def test_pack_output_sizes():
    W = torch.zeros(64, 8)
    with pytest.raises(ValueError, match="bytes"):
        bgb.binarize_pack(W, P=torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="bytes"):    # ternary needs two planes
        bgb.binarize_pack(W, bgb.MODE_TERNARY, P=torch.zeros(bgb.packed_bytes(64, 8) // 4, dtype=torch.int32))


def test_fbi_linear_shapes_dtypes_and_views():
    K, N, M = 64, 8, 2
    P = torch.zeros(bgb.packed_bytes(K, N) // 4, dtype=torch.int32)
    alpha = torch.zeros(N)
    y = torch.zeros(M, N)
    with pytest.raises(ValueError, match="dtype"):                       # fp32 activations
        bgb.fbi_linear_w1a16(torch.zeros(M, K), P, alpha, N, y=y)
    with pytest.raises(ValueError, match="bytes"):                       # P too small
        bgb.fbi_linear_w1a16(bf16(M, K), P[:-1], alpha, N, y=y)
    with pytest.raises(ValueError, match="bytes"):                       # alpha shorter than N
        bgb.fbi_linear_w1a16(bf16(M, K), P, alpha[:N - 1], N, y=y)
    with pytest.raises(ValueError, match="dtype"):                       # bf16 alpha
        bgb.fbi_linear_w1a16(bf16(M, K), P, bf16(N), N, y=y)
    with pytest.raises(ValueError, match="shape"):                       # y of the wrong shape
        bgb.fbi_linear_w1a16(bf16(M, K), P, alpha, N, y=torch.zeros(M, N + 1))
    with pytest.raises(ValueError, match="contiguous"):                  # a transposed view
        bgb.fbi_linear_w1a16(bf16(K, M).t(), P, alpha, N, y=y)


def test_group_items_must_agree():
    M, K, N = 1, 64, 8
    P = torch.zeros(bgb.packed_bytes(K, N) // 4, dtype=torch.int32)
    a32, a16 = torch.zeros(N), torch.zeros(N, dtype=torch.float16)
    item = (bf16(M, K), P, a32, N)
    with pytest.raises(ValueError, match="dtype"):                       # y dtypes differ
        bgb.fbi_linear_w1a16_group([item, item], ys=[torch.zeros(M, N), bf16(M, N)])
    with pytest.raises(ValueError, match="dtype"):                       # alpha dtypes differ
        bgb.fbi_linear_w1a16_group([item, (bf16(M, K), P, a16, N)], ys=[torch.zeros(M, N)] * 2)
    with pytest.raises(ValueError, match="every item"):                  # token counts differ
        bgb.fbi_linear_w1a16_group([item, (bf16(M + 1, K), P, a32, N)], ys=[torch.zeros(M, N)] * 2)
    with pytest.raises(ValueError, match="dtype"):                       # x dtypes differ
        bgb.fbi_linear_w1a16_group([item, (torch.zeros(M, K, dtype=torch.float16), P, a32, N)],
                                   ys=[torch.zeros(M, N)] * 2)
    with pytest.raises(ValueError, match="outputs"):
        bgb.fbi_linear_w1a16_group([item, item], ys=[torch.zeros(M, N)])


def test_bitlinear_argument_checks():
    M, K, N = 3, 64, 8
    P = torch.zeros(bgb.packed_bytes(K, N) // 4, dtype=torch.int32)
    beta = torch.zeros(1)
    with pytest.raises(ValueError, match="dtype"):                       # f16 activations
        bgb.bitlinear_w1a8(torch.zeros(M, K, dtype=torch.float16), P, beta, N)
    with pytest.raises(ValueError, match="shape"):
        bgb.bitlinear_w1a8(torch.zeros(M, K), P, beta, N, y=torch.zeros(M + 1, N))
    with pytest.raises(ValueError, match="bytes"):                       # ternary: two planes
        bgb.bitlinear158_w1a8(torch.zeros(M, K), P, beta, N, y=torch.zeros(M, N))
    with pytest.raises(ValueError, match="dtype"):                       # beta must be fp32
        bgb.bitlinear_w1a8(torch.zeros(M, K), P, bf16(1), N, y=torch.zeros(M, N))
