"""GPU parity: fbi_linear_w1a16_group (several independent FBI-linears; one
launch for a single token) against the fp64 oracle, item by item."""
import numpy as np
import pytest
import torch

import bgb_synth as syn
from gpu_util import check_w1a16, dev_bits16, dev_f32, say, to_bits

pytestmark = pytest.mark.gpu

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

# every block shape of the one-launch form: (pieces per thread, fragments per
# block) = (1, 1), (1, 2), (1, 4), (2, 1), (2, 2), (4, 1); ragged N and K
SHAPES = [(768, 768), (4096, 5000), (1024, 8200), (8192, 300), (6144, 4200), (16384, 100), (96, 65), (11008, 40)]


def _x_bits(x_kind, seed, M, K):
    a = syn.normal_f32(seed, 1, (M, K))
    return syn.f32_to_bf16_bits(a) if x_kind == "bf16" else syn.f32_to_f16_bits(a)


def _items(bgb, shapes, M, x_kind, adt, seed, int_x=False):
    items = []
    for i, (K, N) in enumerate(shapes):
        W = syn.normal_f32(seed + i, 0, (K, N), std=0.02)
        if int_x:
            xf = syn.rng_for(seed + i, 2).integers(-16, 17, size=(M, K)).astype(np.float32)
            xb = syn.f32_to_bf16_bits(xf) if x_kind == "bf16" else syn.f32_to_f16_bits(xf)
        else:
            xb = _x_bits(x_kind, seed + i, M, K)
        if N:
            P, alpha = bgb.binarize_pack(dev_f32(W), bgb.MODE_FBI, TORCH_DT[adt])
        else:
            P, alpha = torch.zeros(4, dtype=torch.int32, device="cuda"), torch.zeros(8, dtype=TORCH_DT[adt],
                                                                                      device="cuda")[:0]
        items.append((W, xb, dev_bits16(xb, TORCH_DT[x_kind]), P, alpha))
    return items


def _check_items(orc, items, ys, x_kind, y_kind, exact=False):
    for (W, xb, _, _, alpha), y in zip(items, ys):
        K, N = W.shape
        if N == 0:
            assert y.shape[1] == 0
            continue
        a_host = alpha.detach().float().cpu().numpy().astype(np.float32)
        ref = orc.fbi_linear(xb, W, a_host, x_kind)
        if exact:
            assert np.array_equal(to_bits(y).astype(np.float32), ref.astype(np.float32)), (K, N)
        else:
            check_w1a16(to_bits(y), ref, y_kind, f"group K={K} N={N}")


@pytest.mark.parametrize("x_kind,adt,y_kind", [("bf16", "f32", "f32"), ("bf16", "f16", "bf16"),
                                               ("f16", "f16", "f16")])
def test_group_single_token_parity(bgb_gpu, orc, x_kind, adt, y_kind):
    say(f"group M=1 {x_kind} alpha={adt} y={y_kind} shapes={SHAPES}")
    items = _items(bgb_gpu, SHAPES, 1, x_kind, adt, 500)
    ys = bgb_gpu.fbi_linear_w1a16_group([(x, P, a, W.shape[1]) for (W, _, x, P, a) in items], TORCH_DT[y_kind])
    torch.cuda.synchronize()
    _check_items(orc, items, ys, x_kind, y_kind)


@pytest.mark.parametrize("x_kind", ["bf16", "f16"])
def test_group_integer_activations_bit_exact(bgb_gpu, orc, x_kind):
    """Integer-valued activations keep every fp32 partial sum exact, so each
    output must equal fl32(alpha * S) whatever block its linear ran in."""
    say(f"group integer-exact {x_kind}")
    items = _items(bgb_gpu, SHAPES, 1, x_kind, "f32", 600, int_x=True)
    ys = bgb_gpu.fbi_linear_w1a16_group([(x, P, a, W.shape[1]) for (W, _, x, P, a) in items])
    torch.cuda.synchronize()
    _check_items(orc, items, ys, x_kind, "f32", exact=True)


@pytest.mark.parametrize("M", [2, 4, 16, 40, 70])
def test_group_several_tokens_parity(bgb_gpu, orc, M):
    """More than one token: one launch for 2..16 tokens (pieces or whole tiles
    staged per item), the grouped GEMM for 17..64 (40), and beyond 64 tokens
    the items one after another through the single-linear GEMM (70)."""
    shapes = [(1024, 300), (11008, 200), (96, 65), (2048, 520)]
    say(f"group M={M} shapes={shapes}")
    items = _items(bgb_gpu, shapes, M, "bf16", "f32", 700 + M)
    ys = bgb_gpu.fbi_linear_w1a16_group([(x, P, a, W.shape[1]) for (W, _, x, P, a) in items], torch.bfloat16)
    torch.cuda.synchronize()
    _check_items(orc, items, ys, "bf16", "bf16")


@pytest.mark.parametrize("M", [4, 8, 16])
@pytest.mark.parametrize("int_x", [True, False])
def test_group_sequential_column_groups(bgb_gpu, orc, M, int_x):
    """2..16 tokens over more column groups than one block per CU can hold at
    the widest groups (378 here): from 8 tokens blocks take several column
    groups one after another on one staging of the tokens, below that the
    grid runs in two rounds. Every output against the oracle; bit-exact on
    integer activations."""
    shapes = [(1024, 24000), (512, 20000), (2048, 4100)]
    say(f"group sequential column groups M={M} int_x={int_x}")
    items = _items(bgb_gpu, shapes, M, "bf16", "f32", 1100 + M, int_x=int_x)
    ys = bgb_gpu.fbi_linear_w1a16_group([(x, P, a, W.shape[1]) for (W, _, x, P, a) in items])
    torch.cuda.synchronize()
    _check_items(orc, items, ys, "bf16", "f32", exact=int_x)


@pytest.mark.parametrize("M", [65, 130, 300])
@pytest.mark.parametrize("int_x", [True, False])
def test_group_prefill_parity(bgb_gpu, orc, M, int_x):
    """More than 64 tokens: the items one after another through the
    single-linear GEMM (a ragged token tile, a K tail, items of different K).
    Every output against the oracle; bit-exact on integer activations."""
    shapes = [(1024, 1000), (2048, 520), (352, 300), (4096, 257)]
    say(f"group prefill M={M} int_x={int_x}")
    items = _items(bgb_gpu, shapes, M, "bf16", "f32", 1200 + M, int_x=int_x)
    ys = bgb_gpu.fbi_linear_w1a16_group([(x, P, a, W.shape[1]) for (W, _, x, P, a) in items])
    torch.cuda.synchronize()
    _check_items(orc, items, ys, "bf16", "f32", exact=int_x)


def test_group_1p3b_layer_prefill_sampled_rows(bgb_gpu, orc):
    """A 1.3B-shaped layer's four fused linears (qkv 2048 x 6144, o 2048 x
    2048, gate_up 2048 x 11264, down 5632 x 2048) over 2048 tokens through
    the group call: 8 sampled token rows of each item against the oracle,
    bf16 outputs."""
    shapes = [(2048, 6144), (2048, 2048), (2048, 11264), (5632, 2048)]
    M = 2048
    say("group 1.3B layer prefill M=2048")
    lin, refs = [], []
    for i, (K, N) in enumerate(shapes):
        W = syn.normal_f32(1300 + i, 0, (K, N), std=0.02)
        xb = _x_bits("bf16", 1300 + i, M, K)
        P, alpha = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_FBI, torch.float16)
        rows = np.sort(syn.rng_for(1300 + i, 4).choice(M, 8, replace=False))
        a_host = alpha.detach().float().cpu().numpy().astype(np.float32)
        refs.append((rows, orc.fbi_linear(np.ascontiguousarray(xb[rows]), W, a_host, "bf16")))
        lin.append((dev_bits16(xb, torch.bfloat16), P, alpha, N))
    ys = bgb_gpu.fbi_linear_w1a16_group(lin, torch.bfloat16)
    torch.cuda.synchronize()
    for (rows, ref), y in zip(refs, ys):
        check_w1a16(to_bits(y)[rows], ref, "bf16", f"1.3B prefill group N={y.shape[1]}")


def test_group_empty_items_and_determinism(bgb_gpu, orc):
    say("group empty items + determinism")
    shapes = [(4096, 300), (1024, 0), (768, 100)]
    items = _items(bgb_gpu, shapes, 1, "bf16", "f32", 800)
    lin = [(x, P, a, W.shape[1]) for (W, _, x, P, a) in items]
    runs = [bgb_gpu.fbi_linear_w1a16_group(lin) for _ in range(4)]
    torch.cuda.synchronize()
    _check_items(orc, items, runs[0], "bf16", "f32")
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)
    assert bgb_gpu.fbi_linear_w1a16_group([]) == []


def test_group_7b_layer_sampled_columns(bgb_gpu, orc):
    """The four same-input-fused linears of a 7B-shaped layer (qkv 4096 x 12288,
    o 4096 x 4096, gate_up 4096 x 22016, down 11008 x 4096) in one launch, as
    the decode benchmark runs them: 96 sampled columns of each against the
    oracle."""
    shapes = [(4096, 12288), (4096, 4096), (4096, 22016), (11008, 4096)]
    say(f"group 7B layer M=1 shapes={shapes}")
    lin, refs = [], []
    for i, (K, N) in enumerate(shapes):
        W = syn.normal_f32(900 + i, 0, (K, N), std=0.02)
        xb = _x_bits("bf16", 900 + i, 1, K)
        P, alpha = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_FBI, torch.float16)
        cols = np.sort(syn.rng_for(900 + i, 3).choice(N, 96, replace=False))
        a_host = alpha.detach().float().cpu().numpy().astype(np.float32)
        refs.append((cols, orc.fbi_linear(xb, np.ascontiguousarray(W[:, cols]), a_host[cols], "bf16")))
        lin.append((dev_bits16(xb, torch.bfloat16), P, alpha, N))
    ys = bgb_gpu.fbi_linear_w1a16_group(lin, torch.bfloat16)
    torch.cuda.synchronize()
    for (cols, ref), y in zip(refs, ys):
        check_w1a16(to_bits(y)[:, cols], ref, "bf16", f"7B group N={y.shape[1]}")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_group_7b_layer_batches_sampled_columns(bgb_gpu, orc, M):
    """The 7B layer's fused linears at 1, 4 and 16 tokens as the decode
    benchmark runs them (at 16 tokens the down projection's tokens do not fit
    in LDS: the other three run as one launch, down alone): 64 sampled columns
    of each item against the oracle."""
    shapes = [(4096, 12288), (4096, 4096), (4096, 22016), (11008, 4096)]
    say(f"group 7B layer M={M}")
    lin, refs = [], []
    for i, (K, N) in enumerate(shapes):
        W = syn.normal_f32(950 + i, 0, (K, N), std=0.02)
        xb = _x_bits("bf16", 950 + i + M, M, K)
        P, alpha = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_FBI, torch.float16)
        cols = np.sort(syn.rng_for(950 + i, 3).choice(N, 64, replace=False))
        a_host = alpha.detach().float().cpu().numpy().astype(np.float32)
        refs.append((cols, orc.fbi_linear(xb, np.ascontiguousarray(W[:, cols]), a_host[cols], "bf16")))
        lin.append((dev_bits16(xb, torch.bfloat16), P, alpha, N))
    ys = bgb_gpu.fbi_linear_w1a16_group(lin, torch.bfloat16)
    torch.cuda.synchronize()
    for (cols, ref), y in zip(refs, ys):
        check_w1a16(to_bits(y)[:, cols], ref, "bf16", f"7B group M={M} N={y.shape[1]}")


def test_group_single_token_beyond_fused_size(bgb_gpu, orc):
    """One item with K beyond the fused single-token size: the other two run
    as one launch, that one alone (the chunked decode)."""
    shapes = [(768, 300), (16416, 40), (4096, 100)]
    say(f"group M=1 sequential shapes={shapes}")
    items = _items(bgb_gpu, shapes, 1, "bf16", "f32", 1000)
    ys = bgb_gpu.fbi_linear_w1a16_group([(x, P, a, W.shape[1]) for (W, _, x, P, a) in items])
    torch.cuda.synchronize()
    _check_items(orc, items, ys, "bf16", "f32")


@pytest.mark.parametrize("M", [2, 3, 8])
def test_group_few_tokens_every_shape(bgb_gpu, orc, M):
    """A few tokens over shapes that take (fragments per block, steps per wave)
    = (8, 8), (4, 4), (4, 1), (2, 4), (2, 2), (1, 4), (1, 1), with ragged N,
    in one launch for M = 2 and 3 (the 12288-row item staging whole tiles at
    M = 3); at M = 8 that item's tokens do not fit in LDS, so the other items
    run as one launch and that one alone."""
    shapes = [(4096, 22016), (4096, 12288), (1024, 8200), (8192, 5000), (4096, 5000), (12288, 100), (96, 65),
              (2048, 300)]
    say(f"group M={M} few-token shapes={shapes}")
    items = _items(bgb_gpu, shapes, M, "bf16", "f16", 1100 + M)
    ys = bgb_gpu.fbi_linear_w1a16_group([(x, P, a, W.shape[1]) for (W, _, x, P, a) in items], torch.bfloat16)
    torch.cuda.synchronize()
    _check_items(orc, items, ys, "bf16", "bf16")


def test_group_few_tokens_integer_bit_exact(bgb_gpu, orc):
    say("group M=4 integer-exact")
    items = _items(bgb_gpu, SHAPES[:6], 4, "bf16", "f32", 1200, int_x=True)
    ys = bgb_gpu.fbi_linear_w1a16_group([(x, P, a, W.shape[1]) for (W, _, x, P, a) in items])
    torch.cuda.synchronize()
    _check_items(orc, items, ys, "bf16", "f32", exact=True)


# ---------------------------------------------------- 17 to 64 tokens ----
# One launch of 64-token x 256-column matrix-core tiles per item, each item's
# K range split into parts whose fp32 sums one reduce launch adds in part
# order.
GEMM_SHAPES = [(2048, 6144), (2048, 2048), (5632, 2048), (96, 65), (352, 300), (4000, 520), (11008, 40),
               (1024, 8200)]


@pytest.mark.parametrize("M", [17, 40, 64])
@pytest.mark.parametrize("x_kind,adt,y_kind", [("bf16", "f16", "bf16"), ("f16", "f32", "f32"),
                                               ("bf16", "f32", "f16")])
def test_group_tokens_17_to_64_parity(bgb_gpu, orc, M, x_kind, adt, y_kind):
    say(f"group M={M} {x_kind} alpha={adt} y={y_kind} shapes={GEMM_SHAPES}")
    items = _items(bgb_gpu, GEMM_SHAPES, M, x_kind, adt, 1300 + M)
    ys = bgb_gpu.fbi_linear_w1a16_group([(x, P, a, W.shape[1]) for (W, _, x, P, a) in items], TORCH_DT[y_kind])
    torch.cuda.synchronize()
    _check_items(orc, items, ys, x_kind, y_kind)


def test_group_tokens_17_to_64_integer_bit_exact(bgb_gpu, orc):
    """Integer activations (|x| <= 16): every partial and split sum is exact
    in fp32, so y = fl32(alpha S) bit for bit."""
    say("group M=33 integer-exact")
    items = _items(bgb_gpu, GEMM_SHAPES, 33, "bf16", "f32", 1400, int_x=True)
    ys = bgb_gpu.fbi_linear_w1a16_group([(x, P, a, W.shape[1]) for (W, _, x, P, a) in items])
    torch.cuda.synchronize()
    _check_items(orc, items, ys, "bf16", "f32", exact=True)


def test_group_tokens_17_to_64_workspace_reuse(bgb_gpu, orc):
    """One workspace (holding stale sums of another group between calls)
    serves repeated calls: results are bit-identical from call to call."""
    say("group M=64 workspace reuse")
    shapes_a = [(2048, 6144), (2048, 2048), (2048, 11264), (5632, 2048)]
    shapes_b = [(4096, 4096), (160, 1000)]
    ia = _items(bgb_gpu, shapes_a, 64, "bf16", "f16", 1500)
    ib = _items(bgb_gpu, shapes_b, 50, "bf16", "f16", 1600)
    la = [(x, P, a, W.shape[1]) for (W, _, x, P, a) in ia]
    lb = [(x, P, a, W.shape[1]) for (W, _, x, P, a) in ib]
    ys_a = [torch.empty((64, W.shape[1]), dtype=torch.bfloat16, device="cuda") for (W, *_) in ia]
    ys_b = [torch.empty((50, W.shape[1]), dtype=torch.bfloat16, device="cuda") for (W, *_) in ib]
    need = max(bgb_gpu.group_workspace_bytes([(x, P, a, y) for (x, P, a, _), y in zip(la, ys_a)], 64),
               bgb_gpu.group_workspace_bytes([(x, P, a, y) for (x, P, a, _), y in zip(lb, ys_b)], 50))
    assert need > 0                                   # the plan splits K for these shapes
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")     # arbitrary prior contents
    first = [y.clone() for y in bgb_gpu.fbi_linear_w1a16_group(la, ys=ys_a, ws=ws)]
    bgb_gpu.fbi_linear_w1a16_group(lb, ys=ys_b, ws=ws)
    for _ in range(3):
        again = bgb_gpu.fbi_linear_w1a16_group(la, ys=ys_a, ws=ws)
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a, b)
    _check_items(orc, ia, first, "bf16", "bf16")
    _check_items(orc, ib, ys_b, "bf16", "bf16")


def test_group_1p3b_fused_layer_decode_b64(bgb_gpu, orc):
    """The four same-input-fused linears of a 1.3B-shaped layer (qkv 2048 x
    6144, o 2048 x 2048, gate_up 2048 x 11264, down 5632 x 2048) for 64 tokens
    in one launch, as the decode benchmark runs them: 128 sampled columns of
    each against the oracle, all 64 tokens."""
    shapes = [(2048, 6144), (2048, 2048), (2048, 11264), (5632, 2048)]
    say(f"group 1.3B fused layer M=64 shapes={shapes}")
    lin, refs = [], []
    for i, (K, N) in enumerate(shapes):
        W = syn.normal_f32(1700 + i, 0, (K, N), std=0.02)
        xb = _x_bits("bf16", 1700 + i, 64, K)
        P, alpha = bgb_gpu.binarize_pack(dev_f32(W), bgb_gpu.MODE_FBI, torch.float16)
        a16 = orc.f32_to_f16(orc.fbi_alpha(W))
        assert np.array_equal(alpha.detach().cpu().view(torch.int16).numpy().view(np.uint16), a16)
        cols = np.sort(syn.rng_for(1700 + i, 3).choice(N, 128, replace=False))
        refs.append((cols, orc.fbi_linear(xb, np.ascontiguousarray(W[:, cols]), orc.f16_to_f32(a16)[cols], "bf16")))
        lin.append((dev_bits16(xb, torch.bfloat16), P, alpha, N))
    ys = bgb_gpu.fbi_linear_w1a16_group(lin, torch.bfloat16)
    torch.cuda.synchronize()
    for (cols, ref), y in zip(refs, ys):
        check_w1a16(to_bits(y)[:, cols], ref, "bf16", f"1.3B group N={y.shape[1]}")
