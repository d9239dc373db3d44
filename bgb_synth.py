"""Seeded synthetic inputs for the binarized linear layers.

This module only draws random tensors and converts storage formats; it holds
none of the layers' arithmetic. Both the device path (through the Python
binding) and the CPU oracle are fed from here, so the two always see
bit-identical inputs.

Conventions
-----------
* Generator: ``numpy.random.default_rng(seed * 1000 + tensor_id)``, then
  ``standard_normal(dtype=float32)`` scaled by ``std`` and shifted by ``mean``
  in float32.
* 16-bit activations are produced from float32 by round-to-nearest-even and
  kept as raw ``uint16`` bit patterns (``bf16`` or ``f16``).
* Weights are float32 ``[K][N]``: row ``i`` is the input feature, column ``j``
  the output feature (``y[M][N] = x[M][K] @ W[K][N]``).
"""
from __future__ import annotations

import hashlib

import numpy as np

__all__ = [
    "rng_for", "normal_f32", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "f32_to_f16_bits", "f16_bits_to_f32", "sha256",
    "LINEAR_SHAPES_7B", "LINEAR_SHAPES_1P3B", "CONFIGS",
]


def rng_for(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(int(seed) * 1000 + int(tensor_id))


def normal_f32(seed: int, tensor_id: int, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    a = rng_for(seed, tensor_id).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return np.ascontiguousarray(a, dtype=np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (NaN stays NaN)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    r = ((u + bias) >> np.uint64(16)).astype(np.uint16)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    r[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def sha256(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


# Linear shapes (K = in features, N = out features) of one decoder layer, in
# layer order q, k, v, o, gate, up, down.
LINEAR_SHAPES_7B = [
    ("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
    ("gate", 4096, 11008), ("up", 4096, 11008), ("down", 11008, 4096),
]
LINEAR_SHAPES_1P3B = [
    ("q", 2048, 2048), ("k", 2048, 2048), ("v", 2048, 2048), ("o", 2048, 2048),
    ("gate", 2048, 5632), ("up", 2048, 5632), ("down", 5632, 2048),
]

# The five workloads: seeds, shapes and distributions.
CONFIGS = {
    "fbi_768": dict(seed=0, K=768, N=768, M=8, w_mean=0.0, w_std=0.02),
    "bitlinear_decode_4096x11008": dict(seed=1, K=4096, N=11008, M=1, w_mean=0.001, w_std=0.02),
    "w1a16_decode_7b_layer": dict(seed=2, shapes=LINEAR_SHAPES_7B, batches=(1, 4, 16), w_std=0.02),
    "w1_prefill_4096x4096x11008": dict(seed=3, M=4096, K=4096, N=11008, w_std=0.02),
    "w1a16_1p3b_stack": dict(seed=4, layers=24, shapes=LINEAR_SHAPES_1P3B, decode_batch=64,
                             prefill_tokens=2048, w_std=0.02),
}


def gpu_normal(seed: int, tensor_id: int, shape, mean: float = 0.0, std: float = 1.0, device="cuda"):
    """Seeded normal float32 tensor drawn directly on the GPU (torch's Philox
    generator seeded with seed * 1000 + tensor_id). Used for the large
    benchmark-only weight stacks, where host generation would dominate setup;
    parity tests use the numpy draws above."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(tensor_id))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t
