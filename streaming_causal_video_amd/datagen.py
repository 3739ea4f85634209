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

from collections import OrderedDict

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_K_OUTLIER, TENSOR_X, TENSOR_W = 0, 1, 2, 3, 4, 5


def _gen(seed: int, stream: int, tensor: int, frame: int) -> np.random.Generator:
    key = np.array([(int(seed) << 16) + int(stream), 0], dtype=np.uint64)
    ctr = np.array([int(tensor), int(frame), 0, 0], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key, counter=ctr))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16, both round-to-nearest-even; returned as fp64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    u += r  # finite inputs only: no carry out of 32 bits
    u &= np.uint32(0xFFFF0000)
    return f.astype(np.float64)


def round_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)


_MEMO: "OrderedDict[tuple, np.ndarray]" = OrderedDict()
_MEMO_BUDGET = 3 << 30  # bytes of generated frames kept for reuse
_memo_bytes = 0


def frame_tensor(w, tensor: int, stream: int, frame: int) -> np.ndarray:
    """One frame of q, k or v for one stream: [P, H, d] fp64 (dtype-exact).

    Generated frames are kept in a small LRU (read-only arrays) so that two
    consumers of the same frame in one process draw it once."""
    global _memo_bytes
    key = (w.seed, w.dtype, w.tokens_per_frame, w.heads, w.head_dim, w.k_outlier_frac, w.k_outlier_scale,
           int(tensor), int(stream), int(frame))
    hit = _MEMO.get(key)
    if hit is not None:
        _MEMO.move_to_end(key)
        return hit
    x = _draw(w, tensor, stream, frame)
    x.setflags(write=False)
    _MEMO[key] = x
    _memo_bytes += x.nbytes
    while _memo_bytes > _MEMO_BUDGET and len(_MEMO) > 1:
        _, old = _MEMO.popitem(last=False)
        _memo_bytes -= old.nbytes
    return x


def _draw(w, tensor: int, stream: int, frame: int) -> np.ndarray:
    shape = (w.tokens_per_frame, w.heads, w.head_dim)
    x = _gen(w.seed, stream, tensor, frame).standard_normal(shape)
    if tensor == TENSOR_K and w.k_outlier_frac > 0.0:
        u = _gen(w.seed, stream, TENSOR_K_OUTLIER, frame).random(shape)
        x[u < w.k_outlier_frac] *= w.k_outlier_scale
    return round_dtype(x, w.dtype)


def frames_tensor(w, tensor: int, t0, n_frames: int) -> np.ndarray:
    """Frames t0[b] .. t0[b]+n_frames-1 of every stream: [B, n*P, H, d]."""
    out = np.empty((w.batch, n_frames * w.tokens_per_frame, w.heads, w.head_dim))
    P = w.tokens_per_frame
    for b in range(w.batch):
        for f in range(n_frames):
            out[b, f * P : (f + 1) * P] = frame_tensor(w, tensor, b, int(t0[b]) + f)
    return out


def hidden_frames(w, d_model: int, t0, n_frames: int) -> np.ndarray:
    """Layer input (hidden states) of frames t0[b] .. t0[b]+n_frames-1:
    [B, n*P, d_model] fp64, N(0, 1) draws rounded to the dtype."""
    P = w.tokens_per_frame
    out = np.empty((w.batch, n_frames * P, d_model))
    for b in range(w.batch):
        for f in range(n_frames):
            x = _gen(w.seed, b, TENSOR_X, int(t0[b]) + f).standard_normal((P, d_model))
            out[b, f * P : (f + 1) * P] = round_dtype(x, w.dtype)
    return out


def qkv_weight(w, d_model: int) -> np.ndarray:
    """Projection weight [3*H*d, d_model] (rows: q features, then k, then v;
    feature h*d + i is dim i of head h): N(0, 1/d_model) draws (unit-variance
    outputs for unit-variance inputs) rounded to the dtype."""
    n_out = 3 * w.heads * w.head_dim
    x = _gen(w.seed, 0, TENSOR_W, 0).standard_normal((n_out, d_model)) / np.sqrt(d_model)
    return round_dtype(x, w.dtype)
