"""Helpers for the GPU parity tests: host<->device moves and the comparison rules.

Comparison rules (tolerances from the stated targets):
* packed words, alpha/beta/c, quantized codes, int32 accumulators: bit-exact;
* W1A16 float outputs: normwise per output row max_j |y - y_ref| / max_j |y_ref|
  <= 2e-3 (fp32 accumulation of exact +-x products against the fp64 oracle);
  16-bit outputs additionally within one unit in the last place of y_ref;
* W1A8 outputs: elementwise |y - y_ref| <= 1e-5 |y_ref| against the fp64
  product acc * beta * gamma / Q_b (acc == 0 gives exactly 0). Where the
  epilogue's scale s = fl32(fl32(beta gamma) / Q_b) or y itself falls below
  FLT_MIN (activations at subnormal scale), each fp32 rounding adds up to
  2^-150 absolute instead of a relative error, so the bound gains
  (|acc| + 1) 2^-149 when the caller passes acc (negligible for normal values).
"""
import sys

import numpy as np
import torch

import bgb_synth as syn

W1A16_NORMWISE_TOL = 2e-3
W1A8_REL_TOL = 1e-5


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_bits16(bits: np.ndarray, dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()
    return t.view(dtype)


def host_u32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint32)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float32)


def host_bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def to_bits(y: torch.Tensor):
    """Device output -> float64 host values."""
    return y.detach().float().cpu().numpy().astype(np.float64)


def normwise_row_err(y: np.ndarray, ref: np.ndarray) -> np.ndarray:
    num = np.max(np.abs(y - ref), axis=1)
    den = np.max(np.abs(ref), axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def check_w1a16(y: np.ndarray, ref: np.ndarray, y_kind: str, tag: str = ""):
    """fp32 outputs: normwise per row <= 2e-3. 16-bit outputs carry one more
    rounding (unit roundoff 2^-8 for bf16, 2^-11 for f16), so each element
    must lie within 2e-3 * rowmax + half an ulp of the fp64 value, and within
    one ulp of it."""
    err = normwise_row_err(y, ref)
    if y_kind == "f32":
        assert np.all(err <= W1A16_NORMWISE_TOL), f"{tag} normwise err {err.max():.3e}"
    else:
        mant = 7 if y_kind == "bf16" else 10
        a = np.abs(ref)
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
        if y_kind == "f16":
            e = np.maximum(e, -14)
        ulp = np.exp2(e - mant)
        rowmax = np.max(np.abs(ref), axis=1, keepdims=True)
        d = np.abs(y - ref)
        bad = d > W1A16_NORMWISE_TOL * rowmax + 0.5 * ulp
        assert not np.any(bad), f"{tag} {int(bad.sum())} outputs beyond 2e-3*rowmax + ulp/2"
        bad1 = d > ulp + 1e-6 * rowmax
        assert not np.any(bad1), f"{tag} {int(bad1.sum())} outputs beyond 1 ulp"
    return float(err.max()) if err.size else 0.0


def check_w1a8(y: np.ndarray, ref: np.ndarray, tag: str = "", acc=None):
    zero = ref == 0
    assert np.all(y[zero] == 0), f"{tag} nonzero output where acc == 0"
    err = np.abs(y[~zero] - ref[~zero])
    if acc is not None:
        floor = (np.abs(np.asarray(acc, np.float64)[~zero]) + 1.0) * 2.0 ** -149
        assert np.all(err <= W1A8_REL_TOL * np.abs(ref[~zero]) + floor), f"{tag} beyond 1e-5 rel + subnormal floor"
        err = np.maximum(err - floor, 0.0)
    rel = err / np.abs(ref[~zero])
    assert rel.size == 0 or rel.max() <= W1A8_REL_TOL, f"{tag} rel err {rel.max():.3e}"
    return float(rel.max()) if rel.size else 0.0


def bf16_input(seed, tid, shape, std=1.0):
    return syn.f32_to_bf16_bits(syn.normal_f32(seed, tid, shape, std=std))
