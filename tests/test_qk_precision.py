"""Why the 14B-shaped layer's rotated q and k are carried in fp16 (CPU only).

That workload scales 1 % of the raw k entries by 30, so scores spread far
wider than with N(0, 1) inputs.  Rounding only the rotated q and k of the
exact oracle computation to bf16 (8 significant bits) already moves the
attention output more than the 1e-2 relative-L2 bar allows; fp16 (11 bits,
same MFMA rate) keeps it well inside.  Everything else here is exact fp64,
so the figures are the floor the storage format alone imposes.  The
rounding helpers live in this test, not in the oracle.
"""
import math

import numpy as np

from oracle import scv_oracle as O
from streaming_causal_video_amd import datagen as G
from streaming_causal_video_amd import workloads as W


def _round_fp16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def _rotated(w, tensor, frames, heads, rows=None):
    """fp64 rotated rows [N, len(heads), d] of stream 0 for the given frames."""
    out = []
    for g in frames:
        x = G.frame_tensor(w, tensor, 0, g)[:, heads]
        t, h, ww = O.token_positions(g, 1, w.grid_h, w.grid_w)
        out.append(O.rope3d(x, t, h, ww, w.split, w.base))
    x = np.concatenate(out, axis=0)
    return x if rows is None else x[rows]


def _floor_errors(w, n_rows=96, heads=(0, 13, 27, 39), seed=0):
    t0 = w.t0[0]
    C = w.chunk_frames
    # the frames the chunk sees: the sink, the window, the chunk itself
    kframes = list(range(w.sink_frames)) + list(range(t0 - w.window_frames, t0 + C))
    heads = list(heads)
    rows = np.sort(np.random.default_rng(seed).choice(C * w.tokens_per_frame, n_rows, replace=False))
    q = _rotated(w, G.TENSOR_Q, range(t0, t0 + C), heads, rows)
    k = _rotated(w, G.TENSOR_K, kframes, heads)
    v = np.concatenate([G.frame_tensor(w, G.TENSOR_V, 0, g)[:, heads] for g in kframes], axis=0)
    scale = 1.0 / math.sqrt(w.head_dim)
    errs = {"bf16": [], "fp16": []}
    for i in range(len(heads)):
        o_ref, _ = O.attention(q[:, i], k[:, i], v[:, i], scale)
        for name, rnd in (("bf16", G.round_bf16), ("fp16", _round_fp16)):
            o, _ = O.attention(rnd(q[:, i]), rnd(k[:, i]), v[:, i], scale)
            errs[name].append((np.linalg.norm(o - o_ref), np.linalg.norm(o_ref)))
    return {n: math.sqrt(sum(a * a for a, _ in e)) / math.sqrt(sum(b * b for _, b in e)) for n, e in errs.items()}


def test_14b_layer_needs_fp16_rotated_operands():
    w = W.WAN14B_480P
    assert w.k_outlier_frac > 0 and w.qk_dtype == "fp16"
    e = _floor_errors(w)
    print(f"rotated q/k rounded to bf16: rel-L2 {e['bf16']:.3e}; to fp16: {e['fp16']:.3e}")
    assert e["bf16"] >= 1e-2, e
    assert e["fp16"] <= 3e-3, e


def test_unit_variance_layer_is_fine_in_bf16():
    """Without the outliers (the 1.3B-shaped layer), bf16 rotated operands
    stay well inside the bar, which is why those workloads keep bf16."""
    w = W.WAN13B_480P
    e = _floor_errors(w, heads=(0, 5, 11))
    print(f"rotated q/k rounded to bf16: rel-L2 {e['bf16']:.3e}; to fp16: {e['fp16']:.3e}")
    assert e["bf16"] <= 3e-3, e
