"""ctypes wrapper around the CPU oracle (``oracle/liboracle.so``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the library's compute path.
Everything here takes and returns numpy arrays on the host.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_sign_fbi.argtypes = [P, I64, I64, P]
    lib.oracle_sign_bitnet.argtypes = [P, I64, I64, ctypes.c_float, P]
    lib.oracle_fbi_alpha.argtypes = [P, I64, I64, P]
    lib.oracle_bitnet_scalars.argtypes = [P, I64, I64, P, P]
    lib.oracle_packed_words.argtypes = [I64, I64]
    lib.oracle_packed_words.restype = I64
    lib.oracle_pack.argtypes = [P, I64, I64, P]
    lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32.restype = ctypes.c_float
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_fbi_linear.argtypes = [P, ctypes.c_int, I64, I64, P, I64, P, P]
    lib.oracle_ln_nonneg_quant.argtypes = [P, I64, I64, ctypes.c_double, ctypes.c_int, ctypes.c_float,
                                           ctypes.c_int, ctypes.c_int, P, P, P]
    lib.oracle_fbi_backward.argtypes = [P, P, ctypes.c_int, I64, I64, P, I64, P, P, P, P]
    lib.oracle_ln_absmax_quant.argtypes = [P, I64, I64, ctypes.c_double, ctypes.c_int,
                                           ctypes.c_float, ctypes.c_int, ctypes.c_int, P, P, P, P]
    lib.oracle_bitlinear_acc.argtypes = [P, I64, I64, P, I64, ctypes.c_float, P]
    lib.oracle_bitlinear_out.argtypes = [P, I64, I64, ctypes.c_float, ctypes.c_float,
                                         ctypes.c_int, P]
    lib.oracle_ternary.argtypes = [P, I64, I64, ctypes.c_float, P, P]
    lib.oracle_int8_acc.argtypes = [P, I64, I64, P, I64, P]
    for name in ("oracle_ternary", "oracle_int8_acc", "oracle_fbi_backward", "oracle_ln_nonneg_quant",
                 "oracle_sign_fbi", "oracle_sign_bitnet", "oracle_fbi_alpha",
                 "oracle_bitnet_scalars", "oracle_pack", "oracle_fbi_linear",
                 "oracle_ln_absmax_quant", "oracle_bitlinear_acc", "oracle_bitlinear_out"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what} rejected its arguments (rc={rc})")


def _f32(W):
    return np.ascontiguousarray(W, dtype=np.float32)


def sign_fbi(W: np.ndarray) -> np.ndarray:
    W = _f32(W)
    K, N = W.shape
    S = np.empty((K, N), np.int8)
    _check(_load().oracle_sign_fbi(_ptr(W), K, N, _ptr(S)), "sign_fbi")
    return S


def sign_bitnet(W: np.ndarray, c: float) -> np.ndarray:
    W = _f32(W)
    K, N = W.shape
    S = np.empty((K, N), np.int8)
    _check(_load().oracle_sign_bitnet(_ptr(W), K, N, ctypes.c_float(c), _ptr(S)), "sign_bitnet")
    return S


def fbi_alpha(W: np.ndarray) -> np.ndarray:
    W = _f32(W)
    K, N = W.shape
    a = np.empty(N, np.float32)
    _check(_load().oracle_fbi_alpha(_ptr(W), K, N, _ptr(a)), "fbi_alpha")
    return a


def bitnet_scalars(W: np.ndarray):
    W = _f32(W)
    K, N = W.shape
    c = np.zeros(1, np.float32)
    b = np.zeros(1, np.float32)
    _check(_load().oracle_bitnet_scalars(_ptr(W), K, N, _ptr(c), _ptr(b)), "bitnet_scalars")
    return np.float32(c[0]), np.float32(b[0])


def packed_words(K: int, N: int) -> int:
    n = _load().oracle_packed_words(K, N)
    if n < 0:
        raise ValueError("K must be a positive multiple of 32")
    return int(n)


def pack(S: np.ndarray) -> np.ndarray:
    S = np.ascontiguousarray(S, dtype=np.int8)
    K, N = S.shape
    P = np.empty(packed_words(K, N), np.uint32)
    _check(_load().oracle_pack(_ptr(S), K, N, _ptr(P)), "pack")
    return P


def f32_to_f16(a: np.ndarray) -> np.ndarray:
    lib = _load()
    flat = np.ascontiguousarray(a, dtype=np.float32).ravel()
    out = np.fromiter((lib.oracle_f32_to_f16(float(v)) for v in flat), dtype=np.uint16, count=flat.size)
    return out.reshape(np.shape(a))


def f16_to_f32(h: np.ndarray) -> np.ndarray:
    lib = _load()
    flat = np.ascontiguousarray(h, dtype=np.uint16).ravel()
    out = np.fromiter((lib.oracle_f16_to_f32(int(v)) for v in flat), dtype=np.float32, count=flat.size)
    return out.reshape(np.shape(h))


def fbi_linear(x_bits: np.ndarray, W: np.ndarray, alpha: np.ndarray, x_kind: str = "bf16") -> np.ndarray:
    """y (fp64) = alpha_j * sum_i sign(W_ij) x_mi for 16-bit activations given as bit patterns."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    W = _f32(W)
    alpha = np.ascontiguousarray(alpha, dtype=np.float32)
    M, K = x_bits.shape
    K2, N = W.shape
    if K2 != K or alpha.shape != (N,):
        raise ValueError("shape mismatch")
    y = np.empty((M, N), np.float64)
    kind = {"bf16": 0, "f16": 1}[x_kind]
    _check(_load().oracle_fbi_linear(_ptr(x_bits), kind, M, K, _ptr(W), N, _ptr(alpha), _ptr(y)),
           "fbi_linear")
    return y


def fbi_backward(x_bits: np.ndarray, dy_bits: np.ndarray, W: np.ndarray, alpha: np.ndarray,
                 x_kind: str = "bf16"):
    """FBI-linear backward through the identity STE: (dX [M][K], dalpha [N], dW [K][N]) in fp64,
    for 16-bit x and dY given as bit patterns of the same kind."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    dy_bits = np.ascontiguousarray(dy_bits, dtype=np.uint16)
    W = _f32(W)
    alpha = np.ascontiguousarray(alpha, dtype=np.float32)
    M, K = x_bits.shape
    K2, N = W.shape
    if K2 != K or alpha.shape != (N,) or dy_bits.shape != (M, N):
        raise ValueError("shape mismatch")
    dx = np.empty((M, K), np.float64)
    da = np.empty(N, np.float64)
    dw = np.empty((K, N), np.float64)
    kind = {"bf16": 0, "f16": 1}[x_kind]
    _check(_load().oracle_fbi_backward(_ptr(x_bits), _ptr(dy_bits), kind, M, K, _ptr(W), N, _ptr(alpha),
                                       _ptr(dx), _ptr(da), _ptr(dw)), "fbi_backward")
    return dx, da, dw


def ln_absmax_quant(x: np.ndarray, ln_eps: float = 1e-5, bits: int = 8, q_eps: float = 1e-3,
                    round_mode: int = 0, gamma_scope: int = 0):
    """Returns (q int8 [M][K], gamma, mu32 [M], rstd32 [M]); gamma is a float32
    scalar for the tensor scope (0) and a float32 [M] array for the token scope (1).
    round_mode 0 truncates toward zero, 1 rounds to nearest even and clamps."""
    x = _f32(x)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    g = np.zeros(max(M, 1), np.float32)
    mu = np.empty(M, np.float32)
    rs = np.empty(M, np.float32)
    _check(_load().oracle_ln_absmax_quant(_ptr(x), M, K, ctypes.c_double(ln_eps), bits,
                                          ctypes.c_float(q_eps), round_mode, gamma_scope, _ptr(q), _ptr(g),
                                          _ptr(mu), _ptr(rs)),
           "ln_absmax_quant")
    gamma = g[:M].copy() if gamma_scope == 1 else np.float32(g[0])
    return q, gamma, mu, rs


def ln_nonneg_quant(x: np.ndarray, ln_eps: float = 1e-5, bits: int = 8, q_eps: float = 1e-3,
                    round_mode: int = 0, gamma_scope: int = 0):
    """eq. (6): returns (q int8 [M][K] in [0, Q_b - 1], gamma, eta); gamma and eta are float32
    scalars for the tensor scope (0) and float32 [M] arrays for the token scope (1)."""
    x = _f32(x)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    g = np.zeros(max(M, 1), np.float32)
    e = np.zeros(max(M, 1), np.float32)
    _check(_load().oracle_ln_nonneg_quant(_ptr(x), M, K, ctypes.c_double(ln_eps), bits, ctypes.c_float(q_eps),
                                          round_mode, gamma_scope, _ptr(q), _ptr(g), _ptr(e)),
           "ln_nonneg_quant")
    if gamma_scope == 1:
        return q, g[:M].copy(), e[:M].copy()
    return q, np.float32(g[0]), np.float32(e[0])


def bitlinear_acc(q: np.ndarray, W: np.ndarray, c: float) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    W = _f32(W)
    M, K = q.shape
    K2, N = W.shape
    if K2 != K:
        raise ValueError("shape mismatch")
    acc = np.empty((M, N), np.int64)
    _check(_load().oracle_bitlinear_acc(_ptr(q), M, K, _ptr(W), N, ctypes.c_float(c), _ptr(acc)),
           "bitlinear_acc")
    return acc


def bitlinear_out(acc: np.ndarray, beta: float, gamma, bits: int = 8) -> np.ndarray:
    """y = acc * beta * gamma / Q_b in fp64; gamma is a scalar or one value per row."""
    acc = np.ascontiguousarray(acc, dtype=np.int64)
    M, N = acc.shape
    y = np.empty((M, N), np.float64)
    g = np.asarray(gamma, np.float32)
    if g.ndim == 0:
        _check(_load().oracle_bitlinear_out(_ptr(acc), M, N, ctypes.c_float(beta), ctypes.c_float(float(g)),
                                            bits, _ptr(y)), "bitlinear_out")
        return y
    for m in range(M):
        row = np.ascontiguousarray(acc[m:m + 1])
        ym = np.empty((1, N), np.float64)
        _check(_load().oracle_bitlinear_out(_ptr(row), 1, N, ctypes.c_float(beta), ctypes.c_float(float(g[m])),
                                            bits, _ptr(ym)), "bitlinear_out")
        y[m] = ym[0]
    return y


# ------------------------------------------------- BitNet b1.58 (ternary) ----

def ternary(W: np.ndarray, eps_w: float = 1e-5):
    """BitNet b1.58 weights ([BitNet] section 二, eq. (9)-(11)): returns
    (T int8 [K][N] in {-1, 0, 1}, gamma_w = mean |W| as float32)."""
    W = _f32(W)
    K, N = W.shape
    T = np.empty((K, N), np.int8)
    g = np.zeros(1, np.float32)
    _check(_load().oracle_ternary(_ptr(W), K, N, ctypes.c_float(eps_w), _ptr(T), _ptr(g)), "ternary")
    return T, np.float32(g[0])


def pack_ternary(T: np.ndarray) -> np.ndarray:
    """Two sign planes in the binary packed format, one after the other: the
    +1 plane, then the -1 plane."""
    T = np.asarray(T)
    return np.concatenate([pack((T > 0).astype(np.int8)), pack((T < 0).astype(np.int8))])


def int8_acc(q: np.ndarray, T: np.ndarray) -> np.ndarray:
    """acc[m][j] = sum_i T[i][j] q[m][i], exact."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    T = np.ascontiguousarray(T, dtype=np.int8)
    M, K = q.shape
    K2, N = T.shape
    if K2 != K:
        raise ValueError("shape mismatch")
    acc = np.empty((M, N), np.int64)
    _check(_load().oracle_int8_acc(_ptr(q), M, K, _ptr(T), N, _ptr(acc)), "int8_acc")
    return acc
