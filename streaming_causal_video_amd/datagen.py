"""Seeded synthetic inputs, shared by tests, the benchmark and the oracle runs.

Values are standard normal fp64 draws from numpy's counter-based Philox
generator, keyed by (seed, stream) and countered by (tensor, frame), so any
frame of any stream can be regenerated on its own.  They are then rounded to
the working dtype: fp64 -> fp32 (round to nearest even), and for bf16 a
further fp32 -> bf16 round to nearest even.  The returned fp64 arrays hold
exactly the values the library receives.

This module contains no RoPE, cache or attention arithmetic.
"""
from __future__ import annotations

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_K_OUTLIER = 0, 1, 2, 3


def _gen(seed: int, stream: int, tensor: int, frame: int) -> np.random.Generator:
    key = np.array([(int(seed) << 16) + int(stream), 0], dtype=np.uint64)
    ctr = np.array([int(tensor), int(frame), 0, 0], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key, counter=ctr))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16, both round-to-nearest-even; returned as fp64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def round_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)


def frame_tensor(w, tensor: int, stream: int, frame: int) -> np.ndarray:
    """One frame of q, k or v for one stream: [P, H, d] fp64 (dtype-exact)."""
    shape = (w.tokens_per_frame, w.heads, w.head_dim)
    x = _gen(w.seed, stream, tensor, frame).standard_normal(shape)
    if tensor == TENSOR_K and w.k_outlier_frac > 0.0:
        u = _gen(w.seed, stream, TENSOR_K_OUTLIER, frame).random(shape)
        x = np.where(u < w.k_outlier_frac, x * w.k_outlier_scale, x)
    return round_dtype(x, w.dtype)


def frames_tensor(w, tensor: int, t0, n_frames: int) -> np.ndarray:
    """Frames t0[b] .. t0[b]+n_frames-1 of every stream: [B, n*P, H, d]."""
    out = np.empty((w.batch, n_frames * w.tokens_per_frame, w.heads, w.head_dim))
    P = w.tokens_per_frame
    for b in range(w.batch):
        for f in range(n_frames):
            out[b, f * P : (f + 1) * P] = frame_tensor(w, tensor, b, int(t0[b]) + f)
    return out
