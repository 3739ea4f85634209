"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bars: fp32 max-abs <= 1e-4, bf16 relative L2 <= 1e-2 (overall and per
stream); fp32 cos/sin tables and slot stamps bit-exact; cached values
bit-exact (they are copied); cached keys within one bf16/fp32 rounding.
Full-size workloads compare every output of the rotation/append and a
sample of attention rows (first/last rows, a tile boundary and random
rows); the smaller cases compare every output.
"""
import numpy as np
import pytest

from oracle import scv_oracle as O
from parity_util import (check_rounding, check_values, compare_tables_bitexact, oracle_replay, record, sample_rows,
                         say, spec_of, to_np)
from streaming_causal_video_amd import datagen as G
from streaming_causal_video_amd import workloads as W
from streaming_causal_video_amd.runner import StreamRunner, to_device

pytestmark = pytest.mark.gpu


def small(name, **kw):
    base = dict(
        name=name, dtype="bf16", batch=1, heads=2, head_dim=128, split=(44, 42, 42), base=10000.0, grid_h=4,
        grid_w=4, chunk_frames=2, sink_frames=1, window_frames=4, t0=(9,), seed=101,
    )
    base.update(kw)
    return W.Workload(**base)


SMALL = [
    small("med-bf16-d128-b2", batch=2, heads=3, grid_h=6, grid_w=10, chunk_frames=3, window_frames=5, t0=(23, 4)),
    small("med-bf16-d64", heads=4, head_dim=64, split=(24, 20, 20), grid_h=5, grid_w=8, sink_frames=2,
          window_frames=3, t0=(11,), seed=102),
    small("med-fp32-d128", dtype="fp32", grid_h=4, grid_w=6, t0=(9,), seed=103),
    small("med-fp32-d64-b3", dtype="fp32", batch=3, head_dim=64, split=(24, 20, 20), grid_h=3, grid_w=8,
          t0=(0, 3, 40), seed=104),
    small("odd-grid-bf16", grid_h=3, grid_w=5, window_frames=3, t0=(7,), seed=105),
    small("odd-grid-fp32", dtype="fp32", head_dim=64, split=(24, 20, 20), grid_h=7, grid_w=3, t0=(12,), seed=106),
    small("multichunk-bf16", grid_h=4, grid_w=8, window_frames=3, max_query_chunks=2, t0=(10,), seed=107),
    small("multichunk3-fp32", dtype="fp32", head_dim=64, split=(24, 20, 20), grid_h=4, grid_w=5,
          window_frames=5, chunk_frames=2, max_query_chunks=3, t0=(14,), seed=108),
    small("no-sink-bf16", sink_frames=0, t0=(9,), seed=109),
    small("warmup-t0-0-bf16", batch=2, t0=(0, 1), seed=110),
    small("max-t0-bf16", t0=((1 << 40) - 2,), seed=111),
    small("long-tiles-bf16", heads=2, grid_h=20, grid_w=26, chunk_frames=2, window_frames=6, t0=(50,), seed=112),
    small("outliers-bf16", grid_h=6, grid_w=8, t0=(30,), k_outlier_frac=0.01, k_outlier_scale=30.0, seed=113),
    small("outliers-qkfp16", grid_h=6, grid_w=8, t0=(30,), k_outlier_frac=0.01, k_outlier_scale=30.0, seed=114,
          qk_dtype="fp16"),
    small("qkfp16-d64-b2", batch=2, heads=3, head_dim=64, split=(24, 20, 20), grid_h=5, grid_w=6, t0=(17, 2),
          qk_dtype="fp16", seed=115),
]


def qk(w):
    return w.qk_dtype or w.dtype


def run_gpu(w, kv_splits=0, fused=True):
    import torch

    r = StreamRunner(w, kv_splits=kv_splits)
    r.fill()
    if fused:
        r.append()
    else:
        q_rot, k_rot = r.cache.rope3d_apply(r.q.clone(), r.k.clone(), w.t0, r.n_frames)
        r.cache.kv_append_roll(k_rot, r.v, w.t0, r.n_frames)
        r.q_rot.copy_(q_rot)
    r.attend()
    torch.cuda.synchronize()
    return r


def check_cache_contents(r, oc, w, heads=None):
    v = r.cache.views()
    stamps = v["stamps"].cpu().numpy()
    assert np.array_equal(stamps, oc.stamps), (stamps, oc.stamps)
    L = r.cache.layout
    P = w.tokens_per_frame
    heads = list(range(w.heads)) if heads is None else heads
    for b in range(w.batch):
        for s in range(w.n_slots):
            if oc.stamps[b, s] < 0:
                continue
            rows = slice(s * L.slot_rows, s * L.slot_rows + P)
            kg = to_np(v["k"][b, heads, rows, :]).transpose(1, 0, 2)
            check_rounding(f"k slot {s}", kg, oc.k[b][s][:, heads], qk(w))
            vg = to_np(v["v_t"][b, heads, :, rows]).transpose(2, 0, 1)
            assert np.array_equal(vg, oc.v[b][s][:, heads]), f"v slot {s} stream {b}"


def check_attention(r, oc, q_rot, w, rows=None, tag=None):
    O_ref, L_ref = oc.chunk_attention(q_rot, w.t0, r.n_frames, rows=rows)
    o = to_np(r.o)
    lse = r.lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        o, lse = o[:, rows], lse[:, :, rows]
    err = check_values("o", o, O_ref, w.dtype, per_axis0=True, tag=tag)
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    if w.dtype == "fp32":
        e = float(np.max(np.abs(lse[fin] - L_ref[fin]))) if fin.any() else 0.0
        say(f"  lse: max-abs {e:.3e}")
        if tag:
            record(case=tag, what="lse", metric="max-abs", value=e)
        assert e <= 1e-4
    else:
        check_values("lse", lse[fin], L_ref[fin], "bf16", tag=tag)
    return err


@pytest.mark.parametrize("w", W.ORDERED + SMALL, ids=lambda w: w.name)
def test_rope_tables_bitexact(w, gpu_lib):
    import torch

    say(f"case tables {w.name}")
    from streaming_causal_video_amd import binding as B

    cache = B.Cache(B.config_for(w))
    cache.cache_init()
    n = w.query_frames
    tabs = cache.rope_tables(w.t0, n)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in tabs.items()}
    skipped = compare_tables_bitexact(got, w.t0, n, w)
    # the static row/column tables held in the cache buffer are the same
    views = cache.views()
    assert np.array_equal(views["table_h"].cpu().numpy().view(np.uint32), got["h"].view(np.uint32))
    assert np.array_equal(views["table_w"].cpu().numpy().view(np.uint32), got["w"].view(np.uint32))
    say(f"  tables bit-exact ({skipped} midpoint entries skipped)")
    record(case=w.name, what="rope tables", metric="bit-exact", value=True, entries=int(sum(v.size for v in got.values())),
           midpoint_skipped=skipped)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_parity_full(w, gpu_lib):
    say(f"case small {w.name}")
    r = run_gpu(w)
    oc, q_rot = oracle_replay(w)
    check_values("q_rot", to_np(r.q_rot), q_rot, w.dtype)
    check_rounding("q_rot", to_np(r.q_rot), q_rot, qk(w))
    check_cache_contents(r, oc, w)
    check_attention(r, oc, q_rot, w)


@pytest.mark.parametrize("w", W.ORDERED, ids=lambda w: w.name)
def test_workload_parity(w, gpu_lib):
    say(f"case workload {w.name}")
    r = run_gpu(w)
    say(f"  gpu done (splits={r.splits}); oracle replay")
    oc, q_rot = oracle_replay(w)
    check_values("q_rot", to_np(r.q_rot), q_rot, w.dtype, per_axis0=True, tag=w.name)
    check_rounding("q_rot", to_np(r.q_rot), q_rot, qk(w))
    heads = sorted({0, w.heads // 2, w.heads - 1})
    check_cache_contents(r, oc, w, heads=heads)
    # the library's own host copy of the stamps agrees with the layout view
    assert np.array_equal(np.array(r.cache.debug_stamps(), dtype=np.int64), oc.stamps)
    record(case=w.name, what="slot stamps", metric="bit-exact", value=True, slots=int(oc.stamps.size))
    rows = None if w.query_rows <= 4096 and w.dtype == "fp32" else sample_rows(w.query_rows, w.seed)
    record(case=w.name, what="o rows compared", metric="count", value=int(w.query_rows if rows is None else len(rows)),
           schedule=int(r.splits))
    check_attention(r, oc, q_rot, w, rows=rows, tag=w.name)


@pytest.mark.parametrize("splits", [2, 3, 7])
def test_split_kv_small(splits, gpu_lib):
    w = SMALL[0]
    say(f"case split {w.name} splits={splits}")
    r = run_gpu(w, kv_splits=splits)
    assert r.splits == splits
    oc, q_rot = oracle_replay(w)
    check_attention(r, oc, q_rot, w)
    r1 = run_gpu(w, kv_splits=1)
    d = np.max(np.abs(to_np(r.o) - to_np(r1.o)))
    say(f"  split vs unsplit max-abs {d:.3e}")
    assert d <= 2.0 ** -7


@pytest.mark.parametrize("splits", [2, 5])
def test_split_kv_multichunk(splits, gpu_lib):
    """Key splits over several query chunks, one of them near the stream
    start (the chunks see different numbers of keys)."""
    w = small("split-multichunk", batch=2, grid_h=4, grid_w=8, window_frames=3, max_query_chunks=3, t0=(2, 40),
              seed=140)
    say(f"case split {w.name} splits={splits}")
    r = run_gpu(w, kv_splits=splits)
    assert r.splits == splits
    oc, q_rot = oracle_replay(w)
    check_attention(r, oc, q_rot, w)


def test_split_kv_720p(gpu_lib):
    w = W.WAN13B_720P
    say(f"case split {w.name} splits=4")
    r = run_gpu(w, kv_splits=4)
    oc, q_rot = oracle_replay(w)
    check_attention(r, oc, q_rot, w, rows=sample_rows(w.query_rows, 7, n_random=96))


BALANCED = [w for w in SMALL if w.dtype == "bf16"] + [
    small("balanced-multichunk", batch=2, grid_h=4, grid_w=8, window_frames=3, max_query_chunks=3, t0=(2, 40),
          seed=141),
    # several query tiles per head (ragged last tile), ranges that cut items
    small("balanced-tiles", heads=3, grid_h=15, grid_w=26, chunk_frames=2, window_frames=4, t0=(31,), seed=142),
]


@pytest.mark.parametrize("w", BALANCED, ids=lambda w: w.name)
def test_balanced_small(w, gpu_lib):
    """The balanced schedule (equal unit ranges, partials merged) against
    the oracle, and against the grid schedule's unsplit output."""
    say(f"case balanced {w.name}")
    r = run_gpu(w, kv_splits=-1)
    assert r.splits == -1
    oc, q_rot = oracle_replay(w)
    check_attention(r, oc, q_rot, w)
    r1 = run_gpu(w, kv_splits=1)
    o1 = to_np(r1.o)
    d = np.max(np.abs(to_np(r.o) - o1))
    say(f"  balanced vs unsplit max-abs {d:.3e}")
    # the merged fp32 partials round to bf16 on their own: outputs may differ
    # by a bf16 rounding step at the largest magnitude (2^-7 relative)
    assert d <= 2.0 ** -7 * max(1.0, float(np.max(np.abs(o1))))


@pytest.mark.parametrize("w", [W.WAN13B_480P_B4, W.WAN14B_480P, W.WAN13B_480P_PREFILL, W.WAN13B_480P_CHUNKS4],
                         ids=lambda w: w.name)
def test_balanced_workloads(w, gpu_lib):
    """Full-size workloads under the balanced schedule (items of different
    lengths, several rounds of ranges), on sampled rows."""
    say(f"case balanced {w.name}")
    r = run_gpu(w, kv_splits=-1)
    say(f"  gpu done (splits={r.splits}); oracle replay")
    assert r.splits == -1
    oc, q_rot = oracle_replay(w)
    check_attention(r, oc, q_rot, w, rows=sample_rows(w.query_rows, w.seed, n_random=48))


ROUNDS = [
    # 16 heads x 17 query tiles = 272 equal items: one round of whole query
    # tiles, then 16 items cut into 256 ranges
    small("rounds-272-items", heads=16, head_dim=64, split=(24, 20, 20), grid_h=40, grid_w=52, chunk_frames=2,
          window_frames=2, t0=(57,), seed=143),
    W.WAN13B_720P,
]


@pytest.mark.parametrize("w", ROUNDS, ids=lambda w: w.name)
def test_rounds_schedule(w, gpu_lib):
    """The balanced schedule with whole-item rounds (kv_splits = -2) against
    the oracle on sampled rows, and against the equal cut."""
    say(f"case rounds {w.name}")
    r = run_gpu(w, kv_splits=-2)
    assert r.splits == -2
    oc, q_rot = oracle_replay(w)
    check_attention(r, oc, q_rot, w, rows=sample_rows(w.query_rows, w.seed, n_random=64))
    r1 = run_gpu(w, kv_splits=-1)
    o1 = to_np(r1.o)
    d = np.max(np.abs(to_np(r.o) - o1))
    say(f"  rounds vs equal cut max-abs {d:.3e}")
    assert d <= 2.0 ** -7 * max(1.0, float(np.max(np.abs(o1))))


def test_side_stream_workspace(gpu_lib):
    """chunk_attention on a side stream with a workspace the binding
    allocates itself, while the default stream allocates and overwrites
    memory right after the call returns: the output equals the default
    stream's (the workspace stays reserved for the side stream until its
    kernels are done)."""
    import torch

    w = small("side-stream", heads=3, grid_h=15, grid_w=26, chunk_frames=2, window_frames=4, t0=(31,), seed=144)
    say(f"case side stream {w.name}")
    r = run_gpu(w, kv_splits=4)
    assert r.splits == 4
    o_ref, lse_ref = r.o.clone(), r.lse.clone()
    need = r.cache.request_workspace_bytes(w.t0, r.n_frames, 4)
    assert need > 0
    side = torch.cuda.Stream()
    o2, lse2 = torch.empty_like(r.o), torch.empty_like(r.lse)
    a = torch.randn(4096, 4096, device="cuda")
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(8):  # keeps the side stream busy past the call's return
            a = (a @ a) * 1e-3
    r.cache.chunk_attention(r.q_rot, w.t0, r.n_frames, o2, lse2, kv_splits=4, stream=side)
    junk = [torch.full((need // 4 + 1,), float("nan"), device="cuda") for _ in range(3)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(o2, o_ref) and torch.equal(lse2, lse_ref)


LIMITS = [
    # 64 frame slots (sink 1 + window 60 + chunk 3), the most the cache
    # accepts: slot masks and ballots use every bit; one stream wraps the
    # ring, one is still filling its window
    small("max-slots-bf16", batch=2, heads=2, grid_h=2, grid_w=4, chunk_frames=3, window_frames=60, t0=(200, 40),
          seed=150),
    small("max-slots-fp32", dtype="fp32", batch=2, heads=2, head_dim=64, split=(24, 20, 20), grid_h=2, grid_w=4,
          chunk_frames=3, window_frames=60, t0=(131, 7), seed=151),
    # 64 streams, the most the kernels' argument blocks hold, each at its own t0
    small("max-batch-bf16", batch=64, heads=1, grid_h=2, grid_w=2, chunk_frames=1, window_frames=2,
          t0=tuple(range(0, 128, 2)), seed=152),
    # 8 query chunks per call, the most a call takes
    small("max-chunks-bf16", grid_h=3, grid_w=4, chunk_frames=2, window_frames=3, max_query_chunks=8, t0=(5,),
          seed=153),
    # 64 streams x 8 chunks: 512 (stream, chunk) classes, a full class table
    small("max-classes-bf16", batch=64, heads=1, grid_h=2, grid_w=2, chunk_frames=1, window_frames=1,
          max_query_chunks=8, t0=tuple(range(0, 192, 3)), seed=154),
]


# the host's choice for every case, and the balanced schedule (bf16 only)
LIMIT_CASES = [(w, 0) for w in LIMITS] + [(w, -1) for w in LIMITS if w.dtype == "bf16"]


@pytest.mark.parametrize("w,kv_splits", LIMIT_CASES, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_size_limits(w, kv_splits, gpu_lib):
    say(f"case limits {w.name} kv_splits={kv_splits}")
    r = run_gpu(w, kv_splits=kv_splits)
    oc, q_rot = oracle_replay(w)
    check_cache_contents(r, oc, w)
    check_attention(r, oc, q_rot, w)


@pytest.mark.parametrize("kv_splits", [-1, 1, 2])
def test_partial_last_chunk(kv_splits, gpu_lib):
    """A call of 3 frames with 2-frame chunks: the second query chunk holds
    one frame (its query tiles are shorter), under every schedule."""
    import torch

    from streaming_causal_video_amd import binding as B

    w = small("ragged-chunk", grid_h=6, grid_w=10, window_frames=3, max_query_chunks=2, t0=(8,), seed=143)
    say(f"case partial last chunk kv_splits={kv_splits}")
    cache = B.Cache(B.config_for(w))
    oc = O.OracleCache(spec_of(w))
    sk, sv = G.frames_tensor(w, G.TENSOR_K, [0], 1), G.frames_tensor(w, G.TENSOR_V, [0], 1)
    cache.cache_init(to_device(sk, "bf16"), to_device(sv, "bf16"))
    oc.init(sk, sv)
    wk, wv = G.frames_tensor(w, G.TENSOR_K, [5], 3), G.frames_tensor(w, G.TENSOR_V, [5], 3)
    cache.rope3d_append(None, None, to_device(wk, "bf16"), to_device(wv, "bf16"), [5], 3)
    oc.kv_append_roll(oc.rope3d_apply(wk, [5], 3), wv, [5], 3)
    n = 3
    q, k, v = (G.frames_tensor(w, t, [8], n) for t in (G.TENSOR_Q, G.TENSOR_K, G.TENSOR_V))
    shape = (1, n * w.tokens_per_frame, w.heads, w.head_dim)
    q_rot = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    o = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, w.heads, shape[1]), dtype=torch.float32, device="cuda")
    cache.rope3d_append(to_device(q, "bf16"), q_rot, to_device(k, "bf16"), to_device(v, "bf16"), [8], n)
    assert cache.attention_splits(n, kv_splits, t0=[8]) == kv_splits
    cache.chunk_attention(q_rot, [8], n, o, lse, kv_splits=kv_splits)
    torch.cuda.synchronize()
    q_ref = oc.rope3d_append(q, k, v, [8], n)
    O_ref, L_ref = oc.chunk_attention(q_ref, [8], n)
    check_values("o", to_np(o), O_ref, "bf16")
    check_values("lse", lse.cpu().numpy().astype(np.float64), L_ref, "bf16")


def test_balanced_empty_cache(gpu_lib):
    """Ranges over a cache with nothing visible: O = 0, lse = -inf."""
    import torch

    from streaming_causal_video_amd import binding as B

    w = small("empty-balanced", grid_h=8, grid_w=8)
    say("case balanced empty cache")
    cache = B.Cache(B.config_for(w))
    cache.cache_init()
    P = w.tokens_per_frame
    shape = (1, 2 * P, 2, 128)
    q = torch.ones(shape, dtype=torch.bfloat16, device="cuda")
    o = torch.full(shape, 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 2, 2 * P), dtype=torch.float32, device="cuda")
    cache.chunk_attention(q, [9], 2, o, lse, kv_splits=-1)
    torch.cuda.synchronize()
    assert torch.all(o == 0)
    assert torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("w", [SMALL[0], SMALL[3], SMALL[4], SMALL[-1]], ids=lambda w: w.name)
def test_unfused_equals_fused(w, gpu_lib):
    import torch

    say(f"case unfused {w.name}")
    a = run_gpu(w, fused=True)
    b = run_gpu(w, fused=False)
    assert torch.equal(a.q_rot, b.q_rot)
    va, vb = a.cache.views(), b.cache.views()
    for name in ("stamps", "table_h", "table_w", "k", "v_t"):
        assert torch.equal(va[name], vb[name]), name
    assert torch.equal(a.o, b.o)


def test_deterministic(gpu_lib):
    import torch

    w = SMALL[0]
    say(f"case determinism {w.name}")
    r = run_gpu(w)
    o1, l1 = r.o.clone(), r.lse.clone()
    r.attend()
    torch.cuda.synchronize()
    assert torch.equal(o1, r.o) and torch.equal(l1, r.lse)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_streaming_many_chunks(dtype, gpu_lib):
    """Stream from t0 = 0 for 30 chunks (several ring wraps), checking every
    chunk's output, the stamps and the cache against the oracle."""
    import torch

    from streaming_causal_video_amd import binding as B

    w = small(f"stream-{dtype}", dtype=dtype, grid_h=4, grid_w=6, window_frames=5, seed=120)
    say(f"case streaming {w.name}")
    cache = B.Cache(B.config_for(w))
    sk = to_device(G.frames_tensor(w, G.TENSOR_K, [0], 1), dtype)
    sv = to_device(G.frames_tensor(w, G.TENSOR_V, [0], 1), dtype)
    cache.cache_init(sk, sv)
    oc = O.OracleCache(spec_of(w))
    oc.init(G.frames_tensor(w, G.TENSOR_K, [0], 1), G.frames_tensor(w, G.TENSOR_V, [0], 1))
    C = w.chunk_frames
    shape = (1, C * w.tokens_per_frame, w.heads, w.head_dim)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for step in range(30):
        t0 = [step * C]
        q = G.frames_tensor(w, G.TENSOR_Q, t0, C)
        k = G.frames_tensor(w, G.TENSOR_K, t0, C)
        v = G.frames_tensor(w, G.TENSOR_V, t0, C)
        q_rot = torch.empty(shape, dtype=tdt, device="cuda")
        o = torch.empty(shape, dtype=tdt, device="cuda")
        lse = torch.empty((1, w.heads, shape[1]), dtype=torch.float32, device="cuda")
        cache.rope3d_append(to_device(q, dtype), q_rot, to_device(k, dtype), to_device(v, dtype), t0, C)
        cache.chunk_attention(q_rot, t0, C, o, lse)
        torch.cuda.synchronize()
        q_ref = oc.rope3d_append(q, k, v, t0, C)
        O_ref, _ = oc.chunk_attention(q_ref, t0, C)
        check_values(f"step {step} o", to_np(o), O_ref, dtype)
        assert np.array_equal(cache.views()["stamps"].cpu().numpy(), oc.stamps)


def test_empty_cache_returns_zero(gpu_lib):
    """A query that sees no key gets O = 0 and lse = -inf."""
    import torch

    from streaming_causal_video_amd import binding as B

    w = small("empty-bf16")
    say("case empty cache")
    cache = B.Cache(B.config_for(w))
    cache.cache_init()
    shape = (1, 2 * 16, 2, 128)
    q = torch.ones(shape, dtype=torch.bfloat16, device="cuda")
    o = torch.full(shape, 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 2, 32), dtype=torch.float32, device="cuda")
    cache.chunk_attention(q, [9], 2, o, lse)
    torch.cuda.synchronize()
    assert torch.all(o == 0)
    assert torch.all(torch.isneginf(lse))


def test_fp16_rotated_keys_saturate(gpu_lib):
    """With fp16 rotated operands, a rotated key beyond +-65504 is stored as
    +-65504 (the documented saturation): the cache holds no inf, and
    attention equals the oracle's attention over keys clamped the same way."""
    import torch

    w = small("fp16-saturate", qk_dtype="fp16", grid_h=4, grid_w=6, t0=(12,), seed=160)
    say(f"case {w.name}")
    r = StreamRunner(w)
    r.fill()
    # first frame of the chunk, head 0: the time dims (and a few others) x 1e5
    P = w.tokens_per_frame
    r.k[0, :P, 0, :8] *= 1.0e5
    r.k[0, :P, 0, 50:54] *= 1.0e5
    r.append()
    r.attend()
    torch.cuda.synchronize()
    k_in = to_np(r.k)

    from parity_util import oracle_fill

    oc = oracle_fill(w)
    nq = w.query_frames
    k_rot = oc.rope3d_apply(k_in, w.t0, nq)
    assert np.max(np.abs(k_rot)) > 65504.0  # the case does saturate
    k_sat = np.clip(k_rot, -65504.0, 65504.0)
    oc.kv_append_roll(k_sat, G.frames_tensor(w, G.TENSOR_V, w.t0, nq), w.t0, nq)
    q_rot = oc.rope3d_apply(G.frames_tensor(w, G.TENSOR_Q, w.t0, nq), w.t0, nq)

    v = r.cache.views()
    slot = w.sink_frames + (w.t0[0] % w.ring_frames)
    L = r.cache.layout
    kc = v["k"][0, :, slot * L.slot_rows: slot * L.slot_rows + P, :].float().cpu().numpy()
    assert np.all(np.isfinite(kc))
    big = np.abs(k_rot[0, :P].transpose(1, 0, 2)) > 65504.0
    assert np.all(np.abs(kc[big]) == 65504.0)
    check_attention(r, oc, q_rot, w)
