"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module only draws and rounds numbers; it holds none of the attention
arithmetic.  Both the float64 oracle and the HIP path consume exactly the arrays
it returns, so the two sides always see bit-identical inputs.

Recipe (one independent PCG64 stream per (seed, b, h), so any subset of heads
can be regenerated on its own):

* draw float64 standard normals for q [N, d], then k [N, d], then v [N, d_v];
* ``normalize=True``: divide every q and k token by its Euclidean norm (the
  unit-sphere inputs the Taylor-state paper uses in its experiments, section 5);
  otherwise multiply q and k by ``scale`` (the unnormalised variant);
* round to float32 (round-to-nearest-even), then, for ``dtype="bf16"``, round
  the float32 values to bfloat16 (round-to-nearest-even) and keep them as
  float32 numbers that are exactly representable in bfloat16.
"""
from __future__ import annotations

import numpy as np

__all__ = ["round_bf16", "bf16_bits", "head_qkv", "make_qkv", "SEEDS"]

# Fixed seeds per workload.
SEEDS = {
    "tiny": 1001,
    "prefill": 1002,
    "decode": 1003,
    "order_sweep": 1004,
    "long": 1005,
    "long_unnormalised": 1006,
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    # NaN stays NaN (quiet), infinities are preserved by the rounding above.
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = np.uint32(0x7FC00000)
    return rounded.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def head_qkv(seed: int, b: int, h: int, N: int, d: int, d_v: int, *,
             normalize: bool = True, scale: float = 1.0, dtype: str = "f32"):
    """q [N,d], k [N,d], v [N,d_v] float32 arrays for one (b, h) stream."""
    rng = np.random.default_rng([int(seed), int(b), int(h)])
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d_v))
    if normalize:
        q = q / np.linalg.norm(q, axis=1, keepdims=True)
        k = k / np.linalg.norm(k, axis=1, keepdims=True)
    else:
        q = q * scale
        k = k * scale
    q = q.astype(np.float32)
    k = k.astype(np.float32)
    v = v.astype(np.float32)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    elif dtype != "f32":
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    return q, k, v


def make_qkv(seed: int, B: int, H: int, N: int, d: int, d_v: int, *,
             normalize: bool = True, scale: float = 1.0, dtype: str = "f32",
             heads=None):
    """Stacked inputs q,k [B,H,N,d], v [B,H,N,d_v] (float32, contiguous).

    ``heads`` optionally restricts generation to a list of (b, h) pairs; the
    other heads are left as zeros (callers fill them some other way).
    """
    q = np.zeros((B, H, N, d), np.float32)
    k = np.zeros((B, H, N, d), np.float32)
    v = np.zeros((B, H, N, d_v), np.float32)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        q[b, h], k[b, h], v[b, h] = head_qkv(seed, b, h, N, d, d_v, normalize=normalize,
                                             scale=scale, dtype=dtype)
    return q, k, v
