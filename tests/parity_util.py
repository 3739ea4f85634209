"""Oracle replay of a workload and comparison helpers for the GPU tests.

The oracle side replays exactly the calls the GPU side makes (cache_init
with the sink frames, the window fill, the fused append of the query chunk)
on the same seeded inputs, then evaluates attention in fp64.
"""
from __future__ import annotations

import json
import sys

import mpmath
import numpy as np

from oracle import scv_oracle as O
from streaming_causal_video_amd import datagen as G
from streaming_causal_video_amd.workloads import Workload, fill_schedule

# Tolerances: fp32 max-abs 1e-4; bf16 relative L2 1e-2.
FP32_MAX_ABS = 1e-4
BF16_REL_L2 = 1e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def spec_of(w: Workload) -> O.CacheSpec:
    return O.CacheSpec(
        batch=w.batch,
        heads=w.heads,
        head_dim=w.head_dim,
        split=w.split,
        base=w.base,
        grid_h=w.grid_h,
        grid_w=w.grid_w,
        sink_frames=w.sink_frames,
        window_frames=w.window_frames,
        chunk_frames=w.chunk_frames,
        max_query_chunks=w.max_query_chunks,
    )


def oracle_fill(w: Workload):
    """OracleCache after the same calls as StreamRunner.fill()."""
    oc = O.OracleCache(spec_of(w))
    if w.sink_frames > 0:
        zeros = [0] * w.batch
        oc.init(G.frames_tensor(w, G.TENSOR_K, zeros, w.sink_frames), G.frames_tensor(w, G.TENSOR_V, zeros, w.sink_frames))
    for starts, n in fill_schedule(w):
        k = G.frames_tensor(w, G.TENSOR_K, starts, n)
        oc.kv_append_roll(oc.rope3d_apply(k, starts, n), G.frames_tensor(w, G.TENSOR_V, starts, n), starts, n)
    return oc


def oracle_replay(w: Workload):
    """OracleCache after the same calls as StreamRunner.fill() + append();
    returns (cache, q_rot fp64)."""
    oc = oracle_fill(w)
    nq = w.query_frames
    q_rot = oc.rope3d_append(
        G.frames_tensor(w, G.TENSOR_Q, w.t0, nq),
        G.frames_tensor(w, G.TENSOR_K, w.t0, nq),
        G.frames_tensor(w, G.TENSOR_V, w.t0, nq),
        w.t0,
        nq,
    )
    return oc, q_rot


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(got, ref) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def record(**fields):
    """One machine-readable result line (collected into the results table of
    the design notes from a run with output shown)."""
    say("PARITY " + json.dumps(fields, sort_keys=True))


def check_values(name, got, ref, dtype, per_axis0=False, tag=None):
    """fp32: max |err| <= 1e-4; bf16: relative L2 <= 1e-2 overall and, with
    per_axis0, per stream; for [B, M, H, d] outputs the worst (stream, head)
    relative L2 is reported too.  Returns the error figure; with tag, records
    the figures."""
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    if dtype == "fp32":
        err = float(np.max(np.abs(got - ref))) if got.size else 0.0
        say(f"  {name}: max-abs {err:.3e}")
        if tag:
            record(case=tag, what=name, metric="max-abs", value=err)
        assert err <= FP32_MAX_ABS, (name, err)
        return err
    err = rel_l2(got, ref)
    per_head = None
    if got.ndim == 4:
        per_head = max(rel_l2(got[b, :, h], ref[b, :, h]) for b in range(got.shape[0]) for h in range(got.shape[2]))
    per_stream = max(rel_l2(got[b], ref[b]) for b in range(got.shape[0])) if per_axis0 else None
    say(f"  {name}: rel-L2 {err:.3e}" + (f", worst (stream, head) {per_head:.3e}" if per_head is not None else ""))
    if tag:
        record(case=tag, what=name, metric="rel-L2", value=err, worst_stream_head=per_head, worst_stream=per_stream)
    assert err <= BF16_REL_L2, (name, err)
    if per_axis0:
        assert per_stream <= BF16_REL_L2, (name, per_stream)
    return err


def check_rounding(name, got, ref, dtype):
    """Element-wise: within one rounding of the storage dtype (plus fp32
    arithmetic), a much tighter check than the L2 bar for pure rotations."""
    # one rounding of the result, plus fp32 rounding of x*c and y*s, which
    # stays absolute when the two products cancel (inputs are O(1)..O(100))
    rel = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11, "fp32": 2.0 ** -22}[dtype]
    bound = rel * np.abs(ref) + 2.0 ** -20 * max(1.0, float(np.max(np.abs(ref))) / 4.0)
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (name, int(bad.sum()), float(np.max(np.abs(got - ref))))


def near_f32_midpoint(x: float) -> bool:
    """Is the exact cos/sin value within 2^-40 (relative) of a float32
    rounding midpoint?  Such entries may round either way legitimately."""
    mpmath.mp.dps = 40
    v = mpmath.mpf(x)
    c = np.float32(x)
    for nb in (np.nextafter(c, np.float32(-np.inf)), np.nextafter(c, np.float32(np.inf))):
        mid = (mpmath.mpf(float(c)) + mpmath.mpf(float(nb))) / 2
        if abs(v - mid) <= abs(v) * mpmath.mpf(2) ** -40:
            return True
    return False


def compare_tables_bitexact(got: dict, t0, n_frames, w: Workload):
    """fp32 cos/sin tables equal the oracle's bit for bit, except entries
    whose exact value sits within 2^-40 of a float32 midpoint (counted)."""
    ref = O.rope_cos_sin_tables(t0, n_frames, w.grid_h, w.grid_w, w.split, w.base)
    skipped = 0
    for key in ("t", "h", "w"):
        g = got[key]
        r = ref[key]
        assert g.shape == r.shape, (key, g.shape, r.shape)
        diff = np.nonzero(g.view(np.uint32) != r.view(np.uint32))
        for idx in zip(*diff):
            # recompute the fp64 angle of this entry and test the midpoint band
            pos_idx, j, cs = idx[:-2], idx[-2], idx[-1]
            d = {"t": w.split[0], "h": w.split[1], "w": w.split[2]}[key]
            if key == "t":
                pos = int(t0[pos_idx[0]]) + int(pos_idx[1])
            else:
                pos = int(pos_idx[0])
            th = O.rope_angles(np.array([pos]), d, w.base)[0, j]
            exact = float(mpmath.cos(mpmath.mpf(th)) if cs == 0 else mpmath.sin(mpmath.mpf(th)))
            assert near_f32_midpoint(exact), (key, idx, g[idx], r[idx])
            skipped += 1
    return skipped


def sample_rows(nq: int, seed: int, n_random=192):
    rng = np.random.default_rng(seed)
    rows = set(range(min(64, nq)))
    rows |= set(range(max(0, 124), min(nq, 132)))
    rows |= set(range(max(0, nq - 70), nq))
    rows |= set(int(x) for x in rng.choice(nq, size=min(n_random, nq), replace=False))
    return np.array(sorted(rows), dtype=np.int64)
