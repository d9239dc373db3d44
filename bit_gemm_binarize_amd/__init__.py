"""Python binding of libbgb.so (binarized linear layers on gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/bgb.h``. torch supplies device
memory and the current stream. If the shared library is missing this module
raises; there is no fallback path.

Entry points mirror the C names:
    binarize_pack(W, mode)            -> packed signs + scales
    fbi_linear_w1a16(x, P, alpha, N)  -> FBI-linear forward (W1A16)
    bitlinear_w1a8(x, P, beta, N)     -> BitLinear forward (W1A8)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

__all__ = [
    "load", "lib_path", "packed_bytes", "MODE_TERNARY", "workspace_bytes", "binarize_pack", "fbi_linear_w1a16",
    "bitlinear_w1a8", "bitlinear_quantize", "bitlinear_matmul", "bitlinear158_w1a8", "bitlinear158_matmul",
    "OP_BITLINEAR158", "BgbError", "QuantParams", "MODE_FBI", "MODE_BITNET",
    "OP_PACK_FBI", "OP_PACK_BITNET", "OP_FBI_LINEAR", "OP_BITLINEAR", "GEMV_MAX_M", "W1A16_DECODE_MAX_M",
    "ROUND_TRUNC", "ROUND_RNE", "GAMMA_TENSOR", "GAMMA_TOKEN", "fbi_linear_w1a16_group", "group_workspace_bytes",
    "GROUP_MAX", "RANGE_SYMMETRIC", "RANGE_NONNEG", "fbi_pack_transposed", "fbi_linear_w1a16_backward", "OP_FBI_BACKWARD",
    "bitlinear_w1a8_noalloc", "noalloc_scratch_bytes", "ESCRATCH",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libbgb.so")

BGB_F32, BGB_F16, BGB_BF16 = 0, 1, 2
MODE_FBI, MODE_BITNET, MODE_TERNARY = 0, 1, 2
OP_PACK_FBI, OP_PACK_BITNET, OP_FBI_LINEAR, OP_BITLINEAR, OP_BITLINEAR158, OP_FBI_BACKWARD = 0, 1, 2, 3, 4, 5
GEMV_MAX_M = 32          # BitLinear: M <= 32 runs the decode kernels, above: the MFMA GEMM
W1A16_DECODE_MAX_M = 64  # FBI-linear: M <= 64 runs the decode kernels, above: the MFMA GEMM
GROUP_MAX = 8            # linears per fbi_linear_w1a16_group call
ESCRATCH = -4            # bitlinear_w1a8_noalloc: the call does not fit the library's static scratch

EXPORTS = ("bgb_packed_bytes", "bgb_workspace_bytes", "binarize_pack", "fbi_linear_w1a16",
           "fbi_linear_w1a16_group", "bgb_group_workspace_bytes", "fbi_pack_transposed",
           "fbi_linear_w1a16_backward",
           "bitlinear_w1a8", "bitlinear_quantize", "bitlinear_matmul", "bitlinear158_w1a8",
           "bitlinear158_matmul", "bitlinear_w1a8_noalloc", "bgb_noalloc_scratch_bytes", "bgb_status_string",
           "bgb_last_hip_error", "bgb_version")


class BgbError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"bgb status {status}: {msg}")
        self.status = status


class _Item(ctypes.Structure):
    """bgb_w1a16_item."""
    _fields_ = [("x", ctypes.c_void_p), ("P", ctypes.c_void_p), ("alpha", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("K", ctypes.c_int64), ("N", ctypes.c_int64)]


class _QP(ctypes.Structure):
    _fields_ = [("ln_eps", ctypes.c_double), ("bits", ctypes.c_int), ("q_eps", ctypes.c_float),
                ("round_mode", ctypes.c_int), ("gamma_scope", ctypes.c_int), ("act_range", ctypes.c_int)]


ROUND_TRUNC, ROUND_RNE = 0, 1
GAMMA_TENSOR, GAMMA_TOKEN = 0, 1
RANGE_SYMMETRIC, RANGE_NONNEG = 0, 1


@dataclass
class QuantParams:
    ln_eps: float = 1e-5
    bits: int = 8
    q_eps: float = 1e-3
    round_mode: int = ROUND_TRUNC
    gamma_scope: int = GAMMA_TENSOR
    act_range: int = RANGE_SYMMETRIC

    def c(self) -> "_QP":
        return _QP(float(self.ln_eps), int(self.bits), float(self.q_eps), int(self.round_mode),
                   int(self.gamma_scope), int(self.act_range))


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libbgb.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m bit_gemm_binarize_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.bgb_packed_bytes.argtypes = [I64, I64]
    lib.bgb_packed_bytes.restype = SZ
    lib.bgb_workspace_bytes.argtypes = [I, I64, I64, I64]
    lib.bgb_workspace_bytes.restype = SZ
    lib.binarize_pack.argtypes = [P, I64, I64, I, P, P, I, P, P, P, SZ, P]
    lib.binarize_pack.restype = I
    lib.fbi_linear_w1a16.argtypes = [P, I, I64, I64, I64, P, P, I, P, I, P, SZ, P]
    lib.fbi_linear_w1a16.restype = I
    lib.fbi_linear_w1a16_group.argtypes = [ctypes.POINTER(_Item), I, I64, I, I, I, P, SZ, P]
    lib.fbi_linear_w1a16_group.restype = I
    lib.bgb_group_workspace_bytes.argtypes = [ctypes.POINTER(_Item), I, I64]
    lib.bgb_group_workspace_bytes.restype = SZ
    lib.fbi_pack_transposed.argtypes = [P, I64, I64, P, P]
    lib.fbi_pack_transposed.restype = I
    lib.fbi_linear_w1a16_backward.argtypes = [P, P, I, I64, I64, I64, P, P, P, I, P, I, P, P, P, SZ, P]
    lib.fbi_linear_w1a16_backward.restype = I
    lib.bitlinear_w1a8.argtypes = [P, I, I64, I64, I64, P, P, ctypes.POINTER(_QP), P, P, P, P, P, SZ, P]
    lib.bitlinear_w1a8.restype = I
    lib.bitlinear_quantize.argtypes = [P, I, I64, I64, ctypes.POINTER(_QP), P, P, P, SZ, P]
    lib.bitlinear_quantize.restype = I
    lib.bitlinear_matmul.argtypes = [I64, I64, I64, P, P, ctypes.POINTER(_QP), P, P, P, SZ, P]
    lib.bitlinear_matmul.restype = I
    lib.bitlinear_w1a8_noalloc.argtypes = [P, I, I64, I64, I64, P, P, ctypes.POINTER(_QP), P, P, P, P, P]
    lib.bitlinear_w1a8_noalloc.restype = I
    lib.bgb_noalloc_scratch_bytes.argtypes = []
    lib.bgb_noalloc_scratch_bytes.restype = SZ
    lib.bitlinear158_w1a8.argtypes = lib.bitlinear_w1a8.argtypes
    lib.bitlinear158_w1a8.restype = I
    lib.bitlinear158_matmul.argtypes = lib.bitlinear_matmul.argtypes
    lib.bitlinear158_matmul.restype = I
    lib.bgb_status_string.argtypes = [I]
    lib.bgb_status_string.restype = ctypes.c_char_p
    lib.bgb_last_hip_error.argtypes = []
    lib.bgb_last_hip_error.restype = I
    lib.bgb_version.argtypes = []
    lib.bgb_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        lib = load()
        msg = lib.bgb_status_string(rc).decode()
        if rc == -3:
            msg += f" (hipError {lib.bgb_last_hip_error()})"
        raise BgbError(rc, msg)


def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    return {torch.float32: BGB_F32, torch.float16: BGB_F16, torch.bfloat16: BGB_BF16}[t.dtype if hasattr(t, "dtype") else t]


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t, name: str, dtypes=None, shape=None, nbytes: int = 0):
    """Reject what the kernels cannot take before any pointer reaches the C ABI:
    a wrong dtype, shape or size, or a non-contiguous view. Raises ValueError.
    Where the tensors live is checked afterwards, for all of a call's tensors
    together (_on_device)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}; expected one of {', '.join(str(d) for d in dtypes)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}; expected {tuple(shape)}")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes; at least {nbytes} are needed")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on_device(device, **tensors):
    """Every tensor handed to the kernels must be a device tensor on the call's
    device (a host pointer would fault the GPU). None entries are skipped."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA (HIP) device tensor, got device {t.device}")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}; the call runs on {device}")


def _f16s():
    torch = _torch()
    return (torch.bfloat16, torch.float16)


def _scales():
    torch = _torch()
    return (torch.float32, torch.float16)


def _ws_ok(ws, device):
    """A caller's workspace: a contiguous device buffer (its size is checked by the library)."""
    if ws is not None:
        _need(ws, "ws")
        _on_device(device, ws=ws)


def _stream(stream) -> Optional[int]:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def packed_bytes(K: int, N: int) -> int:
    return int(load().bgb_packed_bytes(K, N))


def workspace_bytes(op: int, M: int, K: int, N: int) -> int:
    return int(load().bgb_workspace_bytes(op, M, K, N))


def _workspace(op, M, K, N, ws, device):
    _ws_ok(ws, device)
    need = workspace_bytes(op, M, K, N)
    if ws is None:
        torch = _torch()
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return ws


def binarize_pack(W, mode: int = MODE_FBI, alpha_dtype=None, *, P=None, alpha=None, beta=None, centre=None,
                  ws=None, stream=None):
    """W: float32 [K][N] on the GPU. Returns (P, alpha) for FBI or (P, beta, centre) for BitNet
    and ternary (b1.58; beta = mean |W|, P holds the +1 plane then the -1 plane).
    P is an int32 tensor holding the uint32 words of the packed format."""
    torch = _torch()
    if getattr(W, "dim", lambda: 0)() != 2:
        raise ValueError("W must be a 2-D float32 tensor [K][N]")
    K, N = W.shape
    _need(W, "W", (torch.float32,))
    dev = W.device
    planes = 2 if mode == MODE_TERNARY else 1
    if P is None:
        P = torch.empty(max(planes * packed_bytes(K, N) // 4, 4), dtype=torch.int32, device=dev)
    _need(P, "P", nbytes=planes * packed_bytes(K, N))
    for t, nm in ((beta, "beta"), (centre, "centre")):
        if t is not None:
            _need(t, nm, (torch.float32,), nbytes=4)
    op = OP_PACK_FBI if mode == MODE_FBI else OP_PACK_BITNET
    ws = _workspace(op, 0, K, N, ws, dev)
    if mode == MODE_FBI:
        adt = torch.float32 if alpha_dtype is None else alpha_dtype
        if alpha is None:
            alpha = torch.empty(max(N, 8), dtype=adt, device=dev)[:N]
        _need(alpha, "alpha", _scales(), nbytes=N * alpha.element_size())
        _on_device(dev, W=W, P=P, alpha=alpha, ws=ws)
        _check(load().binarize_pack(_ptr(W), K, N, mode, _ptr(P), _ptr(alpha), _dt(alpha), None, None,
                                    _ptr(ws), ws.numel(), _stream(stream)))
        return P, alpha
    if beta is None:
        beta = torch.empty(4, dtype=torch.float32, device=dev)
    if centre is None:
        centre = torch.empty(4, dtype=torch.float32, device=dev)
    _on_device(dev, W=W, P=P, beta=beta, centre=centre, ws=ws)
    _check(load().binarize_pack(_ptr(W), K, N, mode, _ptr(P), None, BGB_F32, _ptr(beta), _ptr(centre),
                                _ptr(ws), ws.numel(), _stream(stream)))
    return P, beta[:1], centre[:1]


def _items(entries):
    arr = (_Item * max(len(entries), 1))()
    for i, (x, P, alpha, y) in enumerate(entries):
        arr[i] = _Item(_ptr(x), _ptr(P), _ptr(alpha), _ptr(y), x.shape[1], y.shape[1])
    return arr


def group_workspace_bytes(entries, M: int) -> int:
    """entries: (x, P, alpha, y) per linear (shapes only are read)."""
    return int(load().bgb_group_workspace_bytes(_items(entries), len(entries), M))


def fbi_linear_w1a16_group(linears, y_dtype=None, *, ys=None, ws=None, stream=None):
    """linears: list of (x, P, alpha, N), x bf16/f16 [M][K] (the same M and dtypes for all).
    Independent linears: one launch for 1 to 64 tokens where the shapes allow it
    (plus one reduce launch when 17..64 tokens split K; see
    fbi_linear_w1a16_group in bgb.h), else one after another. Returns the
    outputs y [M][N]."""
    torch = _torch()
    if not linears:
        return []
    x0 = linears[0][0]
    _need(x0, "x of item 0", _f16s())
    if x0.dim() != 2:
        raise ValueError("x of item 0 must be 2-D [M][K]")
    M = x0.shape[0]
    dev = x0.device
    if ys is None:
        ydt = torch.float32 if y_dtype is None else y_dtype
        ys = [torch.empty((M, N), dtype=ydt, device=dev) for (_, _, _, N) in linears]
    if len(ys) != len(linears):
        raise ValueError(f"{len(ys)} outputs for {len(linears)} linears")
    a0, y0 = linears[0][2], ys[0]
    for i, ((x, P, a, N), y) in enumerate(zip(linears, ys)):
        if x.dim() != 2 or x.shape[0] != M:
            raise ValueError(f"x of item {i} has shape {tuple(x.shape)}; every item needs [{M}][K]")
        K = x.shape[1]
        _need(x, f"x of item {i}", (x0.dtype,))
        _need(P, f"P of item {i}", nbytes=packed_bytes(K, N))
        _need(a, f"alpha of item {i}", (a0.dtype,) if i else _scales(), nbytes=N * a0.element_size())
        _need(y, f"y of item {i}", (y0.dtype,) if i else (torch.float32,) + _f16s(), shape=(M, N))
    entries = [(x, P, a, y) for (x, P, a, _), y in zip(linears, ys)]
    arr = _items(entries)
    _ws_ok(ws, dev)
    need = int(load().bgb_group_workspace_bytes(arr, len(entries), M))
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    for i, ((x, P, a, _), y) in enumerate(zip(linears, ys)):
        _on_device(dev, **{f"x of item {i}": x, f"P of item {i}": P, f"alpha of item {i}": a, f"y of item {i}": y})
    _check(load().fbi_linear_w1a16_group(arr, len(entries), M, _dt(x0), _dt(a0), _dt(y0), _ptr(ws), ws.numel(),
                                         _stream(stream)))
    return ys


def fbi_linear_w1a16(x, P, alpha, N: int, y_dtype=None, *, y=None, ws=None, stream=None):
    """x: bf16/f16 [M][K]; P: packed signs; alpha: [N] f32/f16. Returns y [M][N]."""
    torch = _torch()
    _need(x, "x", _f16s())
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M][K]")
    M, K = x.shape
    dev = x.device
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32 if y_dtype is None else y_dtype, device=dev)
    _need(P, "P", nbytes=packed_bytes(K, N))
    _need(alpha, "alpha", _scales(), nbytes=N * alpha.element_size())
    _need(y, "y", (torch.float32,) + _f16s(), shape=(M, N))
    ws = _workspace(OP_FBI_LINEAR, M, K, N, ws, dev)
    _on_device(dev, x=x, P=P, alpha=alpha, y=y, ws=ws)
    _check(load().fbi_linear_w1a16(_ptr(x), _dt(x), M, K, N, _ptr(P), _ptr(alpha), _dt(alpha), _ptr(y), _dt(y),
                                   _ptr(ws), ws.numel(), _stream(stream)))
    return y


def fbi_pack_transposed(P, K: int, N: int, *, PT=None, stream=None):
    """Packed signs of [S^T; S^T] (2N x K) for the backward product; N % 32 == 0."""
    torch = _torch()
    _need(P, "P", nbytes=packed_bytes(K, N))
    if PT is None:
        PT = torch.empty(max(packed_bytes(2 * N, K) // 4, 4), dtype=torch.int32, device=P.device)
    _need(PT, "PT", nbytes=packed_bytes(2 * N, K))
    _on_device(P.device, P=P, PT=PT)
    _check(load().fbi_pack_transposed(_ptr(P), K, N, _ptr(PT), _stream(stream)))
    return PT


def fbi_linear_w1a16_backward(dy, x, P, PT, alpha, *, want=("dx", "dalpha", "dw"), dx_dtype=None, ws=None,
                              stream=None):
    """FBI-linear backward (identity straight-through estimator). dy: [M][N], x: [M][K] (bf16 or f16,
    the same); P / PT: packed signs and their transposed copy. Returns (dx, dalpha, dw), None for
    what is not in `want`."""
    torch = _torch()
    _need(dy, "dy", _f16s())
    if dy.dim() != 2 or x.dim() != 2 or x.shape[0] != dy.shape[0]:
        raise ValueError(f"dy {tuple(dy.shape)} and x {tuple(x.shape)} must be [M][N] and [M][K]")
    M, N = dy.shape
    K = x.shape[1]
    dev = dy.device
    _need(x, "x", (dy.dtype,))
    _need(P, "P", nbytes=packed_bytes(K, N))
    if "dx" in want:
        _need(PT, "PT", nbytes=packed_bytes(2 * N, K))
    _need(alpha, "alpha", _scales(), nbytes=N * alpha.element_size())
    dx = (torch.empty((M, K), dtype=torch.float32 if dx_dtype is None else dx_dtype, device=dev)
          if "dx" in want else None)
    da = torch.empty(max(N, 4), dtype=torch.float32, device=dev)[:N] if "dalpha" in want else None
    dw = torch.empty((K, N), dtype=torch.float32, device=dev) if "dw" in want else None
    ws = _workspace(OP_FBI_BACKWARD, M, K, N, ws, dev)
    _on_device(dev, dy=dy, x=x, P=P, PT=PT if "dx" in want else None, alpha=alpha, dx=dx, dalpha=da, dw=dw, ws=ws)
    _check(load().fbi_linear_w1a16_backward(_ptr(dy), _ptr(x), _dt(dy), M, K, N, _ptr(P), _ptr(PT), _ptr(alpha),
                                            _dt(alpha), _ptr(dx), _dt(dx) if dx is not None else BGB_F32,
                                            _ptr(da), _ptr(dw), _ptr(ws), ws.numel(), _stream(stream)))
    return dx, da, dw


def bitlinear_w1a8(x, P, beta, N: int, qp: Optional[QuantParams] = None, *, y=None, want_q=False,
                   want_gamma=False, want_acc=False, ws=None, stream=None, _ternary=False):
    """x: f32/bf16 [M][K]; P: packed signs of W - c; beta: device scalar.
    Returns y, or (y, extras) with the requested taps (q, gamma, acc)."""
    torch = _torch()
    _need(x, "x", (torch.float32, torch.bfloat16))
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M][K]")
    M, K = x.shape
    dev = x.device
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    _need(P, "P", nbytes=(2 if _ternary else 1) * packed_bytes(K, N))
    _need(beta, "beta", (torch.float32,), nbytes=4)
    _need(y, "y", (torch.float32,), shape=(M, N))
    qp = qp or QuantParams()
    ng = M if qp.gamma_scope == GAMMA_TOKEN else 1    # gamma: one per token, or one
    q = torch.empty((M, K), dtype=torch.int8, device=dev) if want_q else None
    g = torch.empty(max(ng, 4), dtype=torch.float32, device=dev) if want_gamma else None
    acc = torch.empty((M, N), dtype=torch.int32, device=dev) if want_acc else None
    ws = _workspace(OP_BITLINEAR158 if _ternary else OP_BITLINEAR, M, K, N, ws, dev)
    cqp = qp.c()
    fn = load().bitlinear158_w1a8 if _ternary else load().bitlinear_w1a8
    _on_device(dev, x=x, P=P, beta=beta, y=y, ws=ws)
    _check(fn(_ptr(x), _dt(x), M, K, N, _ptr(P), _ptr(beta), ctypes.byref(cqp), _ptr(y),
                                 _ptr(q), _ptr(g), _ptr(acc), _ptr(ws), ws.numel(), _stream(stream)))
    if not (want_q or want_gamma or want_acc):
        return y
    extras = {}
    if want_q:
        extras["q"] = q
    if want_gamma:
        extras["gamma"] = g[:ng]
    if want_acc:
        extras["acc"] = acc
    return y, extras


def noalloc_scratch_bytes() -> int:
    """Size of the static device array behind bitlinear_w1a8_noalloc."""
    return int(load().bgb_noalloc_scratch_bytes())


def bitlinear_w1a8_noalloc(x, P, beta, N: int, qp: Optional[QuantParams] = None, *, y, q=None, gamma=None,
                           acc=None, stream=None):
    """bitlinear_w1a8 for callers that cannot allocate: the library's static
    device scratch is the workspace and every output is the caller's (y, and
    the optional taps q [M][K] int8, gamma [1] or [M] float32, acc [M][N]
    int32). Nothing is allocated here either. Calls that overlap on one GPU
    race on the shared scratch."""
    torch = _torch()
    _need(x, "x", (torch.float32, torch.bfloat16))
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M][K]")
    M, K = x.shape
    dev = x.device
    qp = qp or QuantParams()
    ng = M if qp.gamma_scope == GAMMA_TOKEN else 1
    _need(P, "P", nbytes=packed_bytes(K, N))
    _need(beta, "beta", (torch.float32,), nbytes=4)
    _need(y, "y", (torch.float32,), shape=(M, N))
    if q is not None:
        _need(q, "q", (torch.int8,), shape=(M, K))
    if gamma is not None:
        _need(gamma, "gamma", (torch.float32,), nbytes=4 * ng)
    if acc is not None:
        _need(acc, "acc", (torch.int32,), shape=(M, N))
    _on_device(dev, x=x, P=P, beta=beta, y=y, q=q, gamma=gamma, acc=acc)
    cqp = qp.c()
    _check(load().bitlinear_w1a8_noalloc(_ptr(x), _dt(x), M, K, N, _ptr(P), _ptr(beta), ctypes.byref(cqp), _ptr(y),
                                         _ptr(q), _ptr(gamma), _ptr(acc), _stream(stream)))
    return y


def bitlinear_quantize(x, qp: Optional[QuantParams] = None, *, ws, N_max: int = 0, want_q=False, want_gamma=False,
                       stream=None):
    """Prologue only: leaves the codes in `ws` for bitlinear_matmul. Returns the requested taps."""
    torch = _torch()
    _need(x, "x", (torch.float32, torch.bfloat16))
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M][K]")
    M, K = x.shape
    _need(ws, "ws")
    qp = qp or QuantParams()
    ng = M if qp.gamma_scope == GAMMA_TOKEN else 1
    q = torch.empty((M, K), dtype=torch.int8, device=x.device) if want_q else None
    g = torch.empty(max(ng, 4), dtype=torch.float32, device=x.device) if want_gamma else None
    cqp = qp.c()
    _on_device(x.device, x=x, ws=ws)
    _check(load().bitlinear_quantize(_ptr(x), _dt(x), M, K, ctypes.byref(cqp), _ptr(q), _ptr(g), _ptr(ws),
                                     ws.numel(), _stream(stream)))
    return {"q": q, "gamma": None if g is None else g[:ng]}


def bitlinear_matmul(M: int, K: int, P, beta, N: int, qp: Optional[QuantParams] = None, *, ws, y=None,
                     want_acc=False, stream=None, _ternary=False):
    """Product + epilogue from the codes a previous bitlinear_quantize left in `ws`."""
    torch = _torch()
    _need(ws, "ws")
    dev = ws.device
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    _need(P, "P", nbytes=(2 if _ternary else 1) * packed_bytes(K, N))
    _need(beta, "beta", (torch.float32,), nbytes=4)
    _need(y, "y", (torch.float32,), shape=(M, N))
    acc = torch.empty((M, N), dtype=torch.int32, device=dev) if want_acc else None
    qp = qp or QuantParams()
    cqp = qp.c()
    fn = load().bitlinear158_matmul if _ternary else load().bitlinear_matmul
    _on_device(dev, P=P, beta=beta, y=y, ws=ws)
    _check(fn(M, K, N, _ptr(P), _ptr(beta), ctypes.byref(cqp), _ptr(y), _ptr(acc), _ptr(ws),
                                   ws.numel(), _stream(stream)))
    return (y, acc) if want_acc else y


def bitlinear158_w1a8(x, P, beta, N: int, qp: Optional[QuantParams] = None, **kw):
    """BitNet b1.58 forward: P holds the two ternary planes from
    binarize_pack(MODE_TERNARY), beta its mean |W|. Same taps as bitlinear_w1a8."""
    return bitlinear_w1a8(x, P, beta, N, qp, _ternary=True, **kw)


def bitlinear158_matmul(M: int, K: int, P, beta, N: int, qp: Optional[QuantParams] = None, **kw):
    """Ternary product + epilogue from the codes a previous bitlinear_quantize left in `ws`."""
    return bitlinear_matmul(M, K, P, beta, N, qp, _ternary=True, **kw)
