"""fp64 CPU oracle: 3D RoPE at a global time index, sink-pinned ring KV cache,
and block-causal chunk attention over sink + window + chunk.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and imports nothing from ``streaming_causal_video_amd``.
It is deliberately plain: numpy in float64, no blocking or fusion beyond what
the definitions below state, so it can be checked against the sources by eye.

Sources, cited by page title and section:

* [SDV2-blog]  "StreamDiffusionV2: A Streaming System for Dynamic and
  Interactive Video Generation" (paper-review blog), section 2 "core idea",
  paragraph on the sink-token guided rolling KV cache: the KV of the initial
  frame(s) is kept as a global anchor (sink), the rest of the cache is a
  fixed-size sliding window, and the RoPE position offset is reset from time
  to time (RoPE refresh).
* [SDV2-summary] "StreamDiffusionV2" (gist.science summary), technical
  summary section 2.A.2 "adaptive sink and RoPE refresh": the same mechanism,
  motivated by positional drift on long streams.
* [CausalRoPE] "Accelerating Video Generation Inference with Sequential-
  Parallel 3D Positional Encoding Using a Global Time Index" (gist.science
  summary), section 2 "methodology": (b) Causal-RoPE SP -- the start frame of
  each generated block serves as the global time index, so every token's time
  position is known locally without communication; (c) cos/sin of the RoPE
  frequencies are precomputed into one contiguous table.  Section 1 names the
  quadratic cost of full spatio-temporal attention and the causal KV cache.

The pages print no formula for RoPE or attention and no worked example.
Readings taken where they are silent:

* R1 pairs are adjacent (2j, 2j+1) inside each axis block (RoPE as a complex
  multiply); R2 each axis a in {t, h, w} is its own 1-D RoPE of width d_a with
  omega_{a,j} = base^(-2j/d_a); R3 axis blocks are contiguous in head_dim in
  the order t, h, w; R4 tokens are frame-major then row-major,
  n = f*P + h*grid_w + w with 0-based h, w; R5 softmax scale 1/sqrt(d);
  R6 sink frames are the stream's first S_f frames (global frames 0..S_f-1);
  R7 the window is the W frames just before the query chunk's start frame;
  R8 block-causal at chunk granularity: a query sees every frame before the
  end of its own chunk, subject to R6/R7; R9 the ring holds
  R = W + max_query_chunks*C frames and frame g >= S_f lives in slot
  S_f + (g mod R); R10 only frames present in the cache are visible (warm-up);
  R11 angles are fp64 products pos*omega, cos/sin are then rounded to fp32;
  R12 a query row that sees no key returns O = 0 and lse = -inf;
  R17 RoPE refresh (the pages' periodic reset of the position offset): the
  time position of frame g of stream b is g - offset[b]; refresh(delta) turns
  the time pairs of every cached key by -delta[b]*omega_t (its time position
  drops by delta[b]) and adds delta[b] to offset[b]; stamps, slots and
  visibility stay on global frame indices, so attention is unchanged in exact
  arithmetic; R18 sink update (the pages' adaptive sink): sink slot j takes
  frame first[b] + j -- its k rotated at that frame's own time position, its
  v, and the frame as stamp -- and the ring is not touched; R19 a key in a
  sink slot is seen by every query chunk that ends after its frame (no
  window rule), a key in a ring slot by R7/R8; R20 the QKV projection that
  the pages fuse with RoPE ([CausalRoPE] 2(c)) is a plain linear map without
  bias or normalisation: q, k, v = x W_q^T, x W_k^T, x W_v^T with one weight
  [3*H*d, d_model] whose rows are the q features, then k, then v (feature
  h*d + i = dim i of head h).

Pinned by tests/test_oracle_*.py (brute force, closed forms, the RoPE
relative-position invariant, torch SDPA in float64, rolling-cache == masked
full-history attention, split/merge identity, hand-computed golden values).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "CacheSpec",
    "rope_frequencies",
    "rope_angles",
    "rope_cos_sin_tables",
    "token_positions",
    "rope3d",
    "frame_slot",
    "frame_visible",
    "slot_visible",
    "attention",
    "merge_partials",
    "qkv_project",
    "OracleCache",
    "full_history_attention",
]


# --------------------------------------------------------------------------
# configuration
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class CacheSpec:
    """Shape of one streaming cache (all streams of a batch share it)."""

    batch: int
    heads: int
    head_dim: int
    split: Tuple[int, int, int]  # (d_t, d_h, d_w), each even, summing to head_dim
    base: float
    grid_h: int
    grid_w: int
    sink_frames: int
    window_frames: int
    chunk_frames: int
    max_query_chunks: int = 1

    @property
    def tokens_per_frame(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def ring_frames(self) -> int:
        # R9: the ring holds the window plus every query chunk of one call.
        return self.window_frames + self.max_query_chunks * self.chunk_frames

    @property
    def n_slots(self) -> int:
        return self.sink_frames + self.ring_frames


# --------------------------------------------------------------------------
# a1 / a2 -- 3D RoPE at a global time index   ([CausalRoPE] 2(b), 2(c);
# [SDV2-blog] 2 RoPE refresh)
# --------------------------------------------------------------------------
def rope_frequencies(d_axis: int, base: float) -> np.ndarray:
    """omega_j = base ** (-2j / d_axis) for j = 0 .. d_axis/2 - 1 (reading R2).

    Each value is one libm ``pow`` call on the fp64 exponent -(2j)/d_axis.
    """
    return np.array(
        [math.pow(float(base), -(2.0 * j) / float(d_axis)) for j in range(d_axis // 2)],
        dtype=np.float64,
    )


def rope_angles(pos, d_axis: int, base: float) -> np.ndarray:
    """theta[..., j] = pos * omega_j as one IEEE fp64 product (reading R11).

    ``pos`` holds integer positions (exact in fp64 below 2**53).
    """
    pos = np.asarray(pos, dtype=np.float64)
    return pos[..., None] * rope_frequencies(d_axis, base)


def rope_cos_sin_tables(
    t0: Sequence[int],
    n_frames: int,
    grid_h: int,
    grid_w: int,
    split: Tuple[int, int, int],
    base: float,
) -> Dict[str, np.ndarray]:
    """The fp32 cos/sin tables the method precomputes ([CausalRoPE] 2(c)).

    Returns float32 arrays with a trailing (cos, sin) axis:
      't': [B, n_frames, d_t/2, 2] at global times t0[b] + f ([CausalRoPE] 2(b)),
      'h': [grid_h, d_h/2, 2] at rows 0..grid_h-1,
      'w': [grid_w, d_w/2, 2] at columns 0..grid_w-1.
    Each entry is float32(cos(theta)) / float32(sin(theta)) of the fp64 angle.
    """
    d_t, d_h, d_w = split
    t_pos = np.asarray(t0, dtype=np.int64)[:, None] + np.arange(n_frames, dtype=np.int64)[None, :]
    out = {}
    for name, pos, width in (
        ("t", t_pos, d_t),
        ("h", np.arange(grid_h, dtype=np.int64), d_h),
        ("w", np.arange(grid_w, dtype=np.int64), d_w),
    ):
        th = rope_angles(pos, width, base)
        out[name] = np.stack([np.cos(th), np.sin(th)], axis=-1).astype(np.float32)
    return out


def token_positions(first_frame, n_frames: int, grid_h: int, grid_w: int):
    """(t, h, w) of every token of frames first_frame .. first_frame+n_frames-1.

    Token order is frame-major then row-major (reading R4); t is the global
    frame index, i.e. the block's start frame plus the frame offset inside the
    block ([CausalRoPE] 2(b)).
    """
    P = grid_h * grid_w
    n = np.arange(n_frames * P, dtype=np.int64)
    f, p = n // P, n % P
    return int(first_frame) + f, p // grid_w, p % grid_w


def rope3d(x: np.ndarray, pos_t, pos_h, pos_w, split: Tuple[int, int, int], base: float) -> np.ndarray:
    """Rotate x [N, H, d] (fp64) by split t/h/w RoPE at per-token positions.

    Head dims [0, d_t) rotate with the time position, [d_t, d_t+d_h) with the
    row, [d_t+d_h, d) with the column (readings R1-R3).  A pair (x, y) at angle
    theta becomes (x cos - y sin, x sin + y cos).
    """
    x = np.asarray(x, dtype=np.float64)
    d_t, d_h, d_w = split
    if d_t + d_h + d_w != x.shape[-1]:
        raise ValueError("split does not sum to head_dim")
    out = np.empty_like(x)
    lo = 0
    for width, pos in ((d_t, pos_t), (d_h, pos_h), (d_w, pos_w)):
        th = rope_angles(pos, width, base)  # [N, width/2]
        c = np.cos(th)[:, None, :]
        s = np.sin(th)[:, None, :]
        xe = x[:, :, lo : lo + width : 2]
        xo = x[:, :, lo + 1 : lo + width : 2]
        out[:, :, lo : lo + width : 2] = xe * c - xo * s
        out[:, :, lo + 1 : lo + width : 2] = xe * s + xo * c
        lo += width
    return out


# --------------------------------------------------------------------------
# a3 -- ring placement and visibility   ([SDV2-blog] 2 sink + rolling cache)
# --------------------------------------------------------------------------
def frame_slot(g: int, sink_frames: int, ring_frames: int) -> int:
    """Cache frame slot of global frame g: sink slot g for the first S_f
    frames (pinned, reading R6), else S_f + (g mod R) (reading R9)."""
    if g < 0:
        raise ValueError("negative frame index")
    return g if g < sink_frames else sink_frames + (g % ring_frames)


def frame_visible(g: int, chunk_start: int, chunk_frames: int, sink_frames: int, window_frames: int) -> bool:
    """May a query in the chunk starting at frame ``chunk_start`` see frame g?

    Block-causal at chunk granularity (R8): g ends before the query chunk
    ends; and g is either a sink frame (R6) or inside the W-frame window just
    before the chunk, or in the chunk itself (R7).
    """
    if g < 0:
        return False
    if g >= chunk_start + chunk_frames:
        return False
    return g < sink_frames or g >= chunk_start - window_frames


def slot_visible(slot: int, g: int, chunk_start: int, chunk_frames: int, sink_frames: int, window_frames: int) -> bool:
    """Visibility of the key held in cache slot ``slot`` (stamped with frame g)
    by slot class (reading R19): sink slots are the global anchor, seen by
    every query chunk that ends after their frame; ring slots follow
    frame_visible.  With the initial frames in the sink (R6) this is exactly
    frame_visible of the slot's frame."""
    if g < 0:
        return False
    if slot < sink_frames:
        return g < chunk_start + chunk_frames
    return frame_visible(g, chunk_start, chunk_frames, sink_frames, window_frames)


# --------------------------------------------------------------------------
# a4 / a5 -- attention and the split/merge identity
# --------------------------------------------------------------------------
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Softmax attention of q [M, d] over k, v [N, d] in fp64.

    S = q k^T * scale; P = softmax(S) row-wise (subtract the row max, exp,
    divide by the row sum); O = P v; lse = max + log(sum exp(S - max)).
    With N = 0 every row returns O = 0 and lse = -inf (reading R12).
    """
    q = np.asarray(q, dtype=np.float64)
    M, d = q.shape
    if k.shape[0] == 0:
        return np.zeros((M, v.shape[1])), np.full(M, -np.inf)
    s = (q @ np.asarray(k, dtype=np.float64).T) * scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e / l) @ np.asarray(v, dtype=np.float64)
    return o, m[:, 0] + np.log(l[:, 0])


def merge_partials(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Combine attention over disjoint key subsets into attention over their
    union: lse = log sum_s exp(lse_s); O = sum_s exp(lse_s - lse) O_s.
    o_parts [S, M, d], lse_parts [S, M]; parts with lse_s = -inf weigh 0."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    lse = np.logaddexp.reduce(lse_parts, axis=0)
    w = np.where(np.isneginf(lse_parts), 0.0, np.exp(lse_parts - np.where(np.isneginf(lse), 0.0, lse)))
    o = (w[..., None] * o_parts).sum(axis=0)
    return o, lse


# --------------------------------------------------------------------------
# QKV projection   ([CausalRoPE] 2(c): fused with RoPE into one kernel)
# --------------------------------------------------------------------------
def qkv_project(x: np.ndarray, w_qkv: np.ndarray, heads: int, head_dim: int):
    """q, k, v [B, N, H, d] of the layer input x [B, N, d_model] under the
    weight w_qkv [3*H*d, d_model] (reading R20), in fp64."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w_qkv, dtype=np.float64).T
    B, N = y.shape[:2]
    y = y.reshape(B, N, 3, heads, head_dim)
    return y[:, :, 0], y[:, :, 1], y[:, :, 2]


# --------------------------------------------------------------------------
# the cache, following the four calls of the boundary
# --------------------------------------------------------------------------
class OracleCache:
    """Slot-indexed model of the sink-pinned ring cache, one per batch.

    Per stream b it keeps ``stamps[b, slot]`` (the global frame a slot holds,
    -1 if empty) and the fp64 rotated keys / values of that frame.  Inputs
    are the exact values the library receives (bf16 or fp32 widened to fp64).
    """

    def __init__(self, spec: CacheSpec):
        self.spec = spec
        self.init()

    # cache_init(sink) -------------------------------------------------------
    def init(self, sink_k: Optional[np.ndarray] = None, sink_v: Optional[np.ndarray] = None):
        """Empty every slot; if given, store the sink frames 0..S_f-1 (raw k,
        rotated here at their global times; [SDV2-blog] 2 sink tokens)."""
        s = self.spec
        self.stamps = np.full((s.batch, s.n_slots), -1, dtype=np.int64)
        # time position of frame g of stream b is g - pos_offset[b] (R17)
        self.pos_offset = np.zeros(s.batch, dtype=np.int64)
        self.k: List[Dict[int, np.ndarray]] = [dict() for _ in range(s.batch)]
        self.v: List[Dict[int, np.ndarray]] = [dict() for _ in range(s.batch)]
        if sink_k is not None:
            zeros = [0] * s.batch
            self.kv_append_roll(self.rope3d_apply(sink_k, zeros, s.sink_frames), sink_v, zeros, s.sink_frames)

    # rope3d_apply(x, t0, grid) ----------------------------------------------
    def rope3d_apply(self, x: np.ndarray, t0: Sequence[int], n_frames: int) -> np.ndarray:
        """Rotate x [B, n_frames*P, H, d]; stream b's frames start at global
        frame t0[b], whose time position is t0[b] - pos_offset[b] (R17)."""
        s = self.spec
        out = np.empty(x.shape, dtype=np.float64)
        for b in range(s.batch):
            t, h, w = token_positions(int(t0[b]) - int(self.pos_offset[b]), n_frames, s.grid_h, s.grid_w)
            out[b] = rope3d(x[b], t, h, w, s.split, s.base)
        return out

    # kv_append_roll(chunk) --------------------------------------------------
    def kv_append_roll(self, k_rot: np.ndarray, v: np.ndarray, t0: Sequence[int], n_frames: int):
        """Write frames t0[b] .. t0[b]+n_frames-1 into their slots (R6, R9),
        evicting whatever each slot held, and stamp the slots."""
        s = self.spec
        P = s.tokens_per_frame
        for b in range(s.batch):
            for f in range(n_frames):
                g = int(t0[b]) + f
                slot = frame_slot(g, s.sink_frames, s.ring_frames)
                self.k[b][slot] = np.array(k_rot[b, f * P : (f + 1) * P], dtype=np.float64)
                self.v[b][slot] = np.array(v[b, f * P : (f + 1) * P], dtype=np.float64)
                self.stamps[b, slot] = g

    def rope3d_append(self, q, k, v, t0, n_frames):
        """Fused form: returns q rotated, appends rotated k and v."""
        self.kv_append_roll(self.rope3d_apply(k, t0, n_frames), v, t0, n_frames)
        return self.rope3d_apply(q, t0, n_frames)

    def qkv_rope_append(self, x, w_qkv, t0, n_frames):
        """Projection of the layer input followed by rope3d_append
        ([CausalRoPE] 2(c)); returns q rotated."""
        q, k, v = qkv_project(x, w_qkv, self.spec.heads, self.spec.head_dim)
        return self.rope3d_append(q, k, v, t0, n_frames)

    # RoPE refresh ([SDV2-blog] 2; [SDV2-summary] 2.A.2) -------------------
    def rope_refresh(self, delta: Sequence[int]):
        """Move stream b's time origin forward by delta[b] frames (R17): every
        cached key -- sink and ring -- has its time pairs turned by
        -delta[b]*omega_t, i.e. it becomes the key rotated at time position
        (its frame - new offset); later rotations of stream b use the new
        offset.  Values, stamps and slots are unchanged."""
        s = self.spec
        for b in range(s.batch):
            dlt = int(delta[b])
            for slot, kk in self.k[b].items():
                n = kk.shape[0]
                zero = np.zeros(n, dtype=np.int64)
                self.k[b][slot] = rope3d(kk, np.full(n, -dlt, dtype=np.int64), zero, zero, s.split, s.base)
            self.pos_offset[b] += dlt

    # sink update ([SDV2-blog] 2; [SDV2-summary] 2.A.2) ----------------------
    def sink_update(self, k: np.ndarray, v: np.ndarray, first_frame: Sequence[int], n_frames: int):
        """Adaptive sink (R18): sink slot j (j < n_frames <= S_f) of stream b
        takes frame first_frame[b] + j -- raw k [B, n_frames*P, H, d] rotated
        at that frame's time position, v as given -- and is stamped with that
        frame.  Ring slots are not touched."""
        s = self.spec
        if not 1 <= n_frames <= s.sink_frames:
            raise ValueError("sink update needs 1 <= n_frames <= sink_frames")
        P = s.tokens_per_frame
        k_rot = self.rope3d_apply(k, first_frame, n_frames)
        for b in range(s.batch):
            for j in range(n_frames):
                self.k[b][j] = np.array(k_rot[b, j * P : (j + 1) * P], dtype=np.float64)
                self.v[b][j] = np.array(v[b, j * P : (j + 1) * P], dtype=np.float64)
                self.stamps[b, j] = int(first_frame[b]) + j

    # chunk_attention(q, cache) -> o ----------------------------------------
    def visible_slots(self, b: int, chunk_start: int) -> List[int]:
        s = self.spec
        return [
            slot
            for slot in range(s.n_slots)
            if self.stamps[b, slot] >= 0
            and slot_visible(slot, int(self.stamps[b, slot]), chunk_start, s.chunk_frames, s.sink_frames,
                             s.window_frames)
        ]

    def chunk_attention(self, q_rot: np.ndarray, t0: Sequence[int], n_frames: int, rows: Optional[np.ndarray] = None):
        """Attention of the query frames t0[b] .. t0[b]+n_frames-1 over the keys
        of the cache that each query may see.

        Query frames are grouped in chunks of C frames from t0[b]; a query of
        chunk c has chunk start t0[b] + c*C.  ``rows`` optionally restricts the
        computation to a subset of query rows (same subset for every stream).
        Returns O [B, M, H, d] and lse [B, H, M].
        """
        s = self.spec
        P, C = s.tokens_per_frame, s.chunk_frames
        n_rows = n_frames * P
        rows = np.arange(n_rows) if rows is None else np.asarray(rows, dtype=np.int64)
        scale = 1.0 / math.sqrt(s.head_dim)
        O = np.zeros((s.batch, rows.size, s.heads, s.head_dim))
        L = np.full((s.batch, s.heads, rows.size), -np.inf)
        chunk_of_row = (rows // P) // C
        for b in range(s.batch):
            for c in np.unique(chunk_of_row):
                sel = np.nonzero(chunk_of_row == c)[0]
                slots = self.visible_slots(b, int(t0[b]) + int(c) * C)
                if slots:
                    K = np.concatenate([self.k[b][sl] for sl in slots], axis=0)
                    V = np.concatenate([self.v[b][sl] for sl in slots], axis=0)
                else:
                    K = np.zeros((0, s.heads, s.head_dim))
                    V = np.zeros((0, s.heads, s.head_dim))
                Q = np.asarray(q_rot[b, rows[sel]], dtype=np.float64)
                for hh in range(s.heads):
                    o, lse = attention(Q[:, hh], K[:, hh], V[:, hh], scale)
                    O[b, sel, hh] = o
                    L[b, hh, sel] = lse
        return O, L


def full_history_attention(
    spec: CacheSpec,
    q_rot: np.ndarray,
    k_rot_frames: Dict[int, np.ndarray],
    v_frames: Dict[int, np.ndarray],
    chunk_start: int,
):
    """Attention of one query chunk (q_rot [M, H, d]) over the full history of
    frames 0 .. chunk_start+C-1 with an explicit 0/1 mask that keeps only the
    sink frames and the W-frame window (the definition the rolling cache must
    reproduce).  ``k_rot_frames[g]`` / ``v_frames[g]`` are [P, H, d]."""
    end = chunk_start + spec.chunk_frames
    frames = [g for g in range(end) if g in k_rot_frames]
    K = np.concatenate([k_rot_frames[g] for g in frames], axis=0)
    V = np.concatenate([v_frames[g] for g in frames], axis=0)
    key_frame = np.repeat(np.array(frames), spec.tokens_per_frame)
    mask = np.array(
        [frame_visible(int(g), chunk_start, spec.chunk_frames, spec.sink_frames, spec.window_frames) for g in key_frame]
    )
    scale = 1.0 / math.sqrt(spec.head_dim)
    M = q_rot.shape[0]
    O = np.zeros((M, spec.heads, spec.head_dim))
    L = np.zeros((spec.heads, M))
    for hh in range(spec.heads):
        s = (q_rot[:, hh] @ K[:, hh].T) * scale
        s = np.where(mask[None, :], s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        O[:, hh] = (e / l) @ V[:, hh]
        L[hh] = m[:, 0] + np.log(l[:, 0])
    return O, L
