"""GPU parity of RoPE refresh and sink update (through the C ABI) against the
fp64 oracle.

Bars as elsewhere: bf16 relative L2 <= 1e-2 (fp32 max-abs <= 1e-4) for
outputs and cached keys; stamps, time offsets and untouched cache regions
bit-exact; a freshly rotated sink key within one rounding of the key dtype.
A refresh changes outputs only by rounding, so the output after a refresh is
also compared with the output before it.
"""
import numpy as np
import pytest

from oracle import scv_oracle as O
from parity_util import check_rounding, check_values, oracle_replay, sample_rows, say, spec_of, to_np
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


REFRESH_CASES = [
    small("refresh-bf16-b2", batch=2, heads=3, grid_h=6, grid_w=10, chunk_frames=3, window_frames=5, t0=(230, 40),
          seed=201),
    small("refresh-fp32-d64", dtype="fp32", head_dim=64, split=(24, 20, 20), grid_h=5, grid_w=7, t0=(77,), seed=202),
    small("refresh-qkfp16", grid_h=6, grid_w=8, t0=(3000,), qk_dtype="fp16", seed=203),
    small("refresh-multichunk", grid_h=4, grid_w=8, window_frames=3, max_query_chunks=2, sink_frames=2,
          t0=(1 << 30,), seed=204),
]


def qk(w):
    return w.qk_dtype or w.dtype


def cache_keys(r, oc, w, heads=None):
    """(gpu, oracle) key arrays over every stamped slot: [n, heads, d]."""
    v = r.cache.views()
    L = r.cache.layout
    P = w.tokens_per_frame
    heads = list(range(w.heads)) if heads is None else heads
    got, ref = [], []
    for b in range(w.batch):
        for s in range(w.n_slots):
            if oc.stamps[b, s] < 0:
                continue
            rows = slice(s * L.slot_rows, s * L.slot_rows + P)
            got.append(to_np(v["k"][b, heads, rows, :]).transpose(1, 0, 2))
            ref.append(oc.k[b][s][:, heads])
    return np.concatenate(got), np.concatenate(ref)


def attention_check(r, oc, q_ref, w, rows=None):
    O_ref, L_ref = oc.chunk_attention(q_ref, w.t0, r.n_frames, rows=rows)
    o = to_np(r.o)
    lse = r.lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        o, lse = o[:, rows], lse[:, :, rows]
    check_values("o", o, O_ref, w.dtype, per_axis0=True)
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    check_values("lse", lse[fin], L_ref[fin], "fp32" if w.dtype == "fp32" else "bf16")
    return O_ref


def refresh_deltas(w):
    # move each stream's current chunk to time position S_f + W (keeps every
    # later position >= 0); a stream already there is left alone (delta 0)
    return [max(0, t - (w.sink_frames + w.window_frames)) for t in w.t0]


def run_refresh_case(w, rows=None, heads=None):
    import torch

    r = StreamRunner(w)
    r.fill()
    r.step()
    torch.cuda.synchronize()
    o_before = to_np(r.o)
    vt_before = r.cache.views()["v_t"].clone()
    stamps_before = r.cache.views()["stamps"].clone()
    oc, q_ref = oracle_replay(w)
    delta = refresh_deltas(w)
    say(f"  refresh by {delta}")
    r.cache.rope_refresh(delta)
    oc.rope_refresh(delta)
    torch.cuda.synchronize()
    assert r.cache.time_offsets() == delta
    v = r.cache.views()
    assert torch.equal(v["stamps"], stamps_before)
    assert torch.equal(v["v_t"], vt_before)  # values untouched
    kg, kr = cache_keys(r, oc, w, heads)
    check_values("k after refresh", kg, kr, w.dtype)
    # the same chunk again: q and k now rotate at (frame - offset)
    r.step()
    torch.cuda.synchronize()
    q_ref = oc.rope3d_append(
        G.frames_tensor(w, G.TENSOR_Q, w.t0, r.n_frames),
        G.frames_tensor(w, G.TENSOR_K, w.t0, r.n_frames),
        G.frames_tensor(w, G.TENSOR_V, w.t0, r.n_frames),
        w.t0,
        r.n_frames,
    )
    check_values("q_rot after refresh", to_np(r.q_rot), q_ref, w.dtype)
    attention_check(r, oc, q_ref, w, rows=rows)
    o_after = to_np(r.o)
    if rows is not None:
        o_before, o_after = o_before[:, rows], o_after[:, rows]
    check_values("o after vs before refresh", o_after, o_before, w.dtype)


@pytest.mark.parametrize("w", REFRESH_CASES, ids=lambda w: w.name)
def test_refresh_parity(w, gpu_lib):
    say(f"case refresh {w.name}")
    run_refresh_case(w)


def test_refresh_parity_480p(gpu_lib):
    w = W.WAN13B_480P
    say(f"case refresh {w.name}")
    run_refresh_case(w, rows=sample_rows(w.query_rows, 31, n_random=96), heads=[0, w.heads - 1])


def test_refresh_zero_delta_is_a_no_op(gpu_lib):
    import torch

    w = REFRESH_CASES[0]
    say(f"case refresh-zero {w.name}")
    r = StreamRunner(w)
    r.fill()
    torch.cuda.synchronize()
    k0 = r.cache.views()["k"].clone()
    r.cache.rope_refresh([0] * w.batch)
    torch.cuda.synchronize()
    assert torch.equal(r.cache.views()["k"], k0)
    # one stream refreshed, the other untouched bit for bit
    r.cache.rope_refresh([5, 0])
    torch.cuda.synchronize()
    k1 = r.cache.views()["k"]
    assert torch.equal(k1[1], k0[1]) and not torch.equal(k1[0], k0[0])
    assert r.cache.time_offsets() == [5, 0]


def test_refresh_rejects_negative_positions(gpu_lib):
    import torch

    from streaming_causal_video_amd import binding as B

    w = REFRESH_CASES[1]
    say(f"case refresh-range {w.name}")
    r = StreamRunner(w)
    r.fill()
    r.cache.rope_refresh([70])
    torch.cuda.synchronize()
    with pytest.raises(B.ScvError) as e:
        r.cache.rope3d_append(r.q, r.q_rot, r.k, r.v, [60], r.n_frames)
    assert e.value.status == -5
    r.cache.cache_init()  # resets the offsets
    assert r.cache.time_offsets() == [0]


SINK_CASES = [
    small("sink-bf16-b2", batch=2, heads=3, grid_h=6, grid_w=10, chunk_frames=3, window_frames=5, t0=(230, 40),
          seed=211),
    small("sink2-fp32-d64", dtype="fp32", head_dim=64, split=(24, 20, 20), grid_h=5, grid_w=7, sink_frames=2,
          window_frames=3, t0=(77,), seed=212),
    small("sink-qkfp16", grid_h=6, grid_w=8, t0=(3000,), qk_dtype="fp16", seed=213),
]


def sink_update_case(w, first_in_call, n_sink, rows=None):
    """After the step, the sink takes frames t0 + first_in_call .. of the
    call's own k/v; attention of the same chunk is checked again."""
    import torch

    r = StreamRunner(w)
    r.fill()
    r.step()
    torch.cuda.synchronize()
    oc, q_ref = oracle_replay(w)
    P = w.tokens_per_frame
    v_before = r.cache.views()
    L = r.cache.layout
    ring_rows = slice(w.sink_frames * L.slot_rows, None)
    k_ring = v_before["k"][:, :, ring_rows].clone()
    vt_ring = v_before["v_t"][:, :, :, ring_rows].clone()
    sel = slice(first_in_call * P, (first_in_call + n_sink) * P)
    k_new = r.k[:, sel].contiguous()
    v_new = r.v[:, sel].contiguous()
    first = [t + first_in_call for t in w.t0]
    say(f"  sink <- frames {first} (+{n_sink})")
    r.cache.sink_update(k_new, v_new, first, n_sink)
    oc.sink_update(G.frames_tensor(w, G.TENSOR_K, first, n_sink), G.frames_tensor(w, G.TENSOR_V, first, n_sink),
                   first, n_sink)
    r.attend()
    torch.cuda.synchronize()
    v = r.cache.views()
    assert np.array_equal(v["stamps"].cpu().numpy(), oc.stamps)
    assert torch.equal(v["k"][:, :, ring_rows], k_ring) and torch.equal(v["v_t"][:, :, :, ring_rows], vt_ring)
    for b in range(w.batch):
        for s in range(n_sink):
            rws = slice(s * L.slot_rows, s * L.slot_rows + P)
            kg = to_np(v["k"][b, :, rws, :]).transpose(1, 0, 2)
            check_rounding(f"sink {s} k", kg, oc.k[b][s], qk(w))
            vg = to_np(v["v_t"][b, :, :, rws]).transpose(2, 0, 1)
            assert np.array_equal(vg, oc.v[b][s])
    attention_check(r, oc, q_ref, w, rows=rows)


@pytest.mark.parametrize("w", SINK_CASES, ids=lambda w: w.name)
def test_sink_update_parity(w, gpu_lib):
    say(f"case sink {w.name}")
    sink_update_case(w, 0, w.sink_frames)


def test_sink_update_hidden_from_earlier_chunk(gpu_lib):
    """Two query chunks; the sink takes a frame of the second chunk, which the
    first chunk must not see (block-causal), while the second chunk does."""
    w = small("sink-multichunk", grid_h=4, grid_w=8, window_frames=3, max_query_chunks=2, t0=(50,), seed=214)
    say(f"case sink {w.name}")
    sink_update_case(w, w.chunk_frames + 1, 1)


def test_sink_update_480p(gpu_lib):
    w = W.WAN13B_480P
    say(f"case sink {w.name}")
    sink_update_case(w, w.chunk_frames - 1, 1, rows=sample_rows(w.query_rows, 33, n_random=96))


def append_sink_case(w, sink_first, n_sink, rows=None):
    """rope3d_append with a sink update from the same chunk in one launch:
    bit-exact against the two separate calls, and against the oracle's
    rope3d_append followed by its sink_update."""
    import torch

    P = w.tokens_per_frame
    fused = StreamRunner(w)
    fused.fill()
    fused.cache.rope3d_append_sink(fused.q, fused.q_rot, fused.k, fused.v, list(w.t0), w.query_frames, sink_first,
                                   n_sink)
    sep = StreamRunner(w)
    sep.fill()
    sep.append()
    sel = slice(sink_first * P, (sink_first + n_sink) * P)
    first = [t + sink_first for t in w.t0]
    sep.cache.sink_update(sep.k[:, sel].contiguous(), sep.v[:, sel].contiguous(), first, n_sink)
    torch.cuda.synchronize()
    vf, vs = fused.cache.views(), sep.cache.views()
    for key in ("k", "v_t", "stamps"):
        assert torch.equal(vf[key], vs[key]), key
    assert torch.equal(fused.q_rot, sep.q_rot)
    oc, q_ref = oracle_replay(w)
    oc.sink_update(G.frames_tensor(w, G.TENSOR_K, first, n_sink), G.frames_tensor(w, G.TENSOR_V, first, n_sink),
                   first, n_sink)
    assert np.array_equal(vf["stamps"].cpu().numpy(), oc.stamps)
    L = fused.cache.layout
    for b in range(w.batch):
        for s in range(n_sink):
            rws = slice(s * L.slot_rows, s * L.slot_rows + P)
            check_rounding(f"sink {s} k", to_np(vf["k"][b, :, rws, :]).transpose(1, 0, 2), oc.k[b][s], qk(w))
            assert np.array_equal(to_np(vf["v_t"][b, :, :, rws]).transpose(2, 0, 1), oc.v[b][s])
    fused.attend()
    torch.cuda.synchronize()
    attention_check(fused, oc, q_ref, w, rows=rows)


APPEND_SINK_CASES = [
    (small("append-sink-b2", batch=2, heads=3, grid_h=6, grid_w=10, chunk_frames=3, window_frames=5, t0=(230, 40),
           sink_frames=2, seed=221), 1, 2),
    (small("append-sink-fp32", dtype="fp32", head_dim=64, split=(24, 20, 20), grid_h=5, grid_w=7, t0=(77,),
           seed=222), 1, 1),
    (small("append-sink-qkfp16", grid_h=6, grid_w=8, t0=(3000,), qk_dtype="fp16", seed=223), 0, 1),
    (small("append-sink-odd-grid", grid_h=3, grid_w=5, chunk_frames=3, t0=(12,), seed=224), 2, 1),
]


@pytest.mark.parametrize("w,first,n", APPEND_SINK_CASES, ids=[c[0].name for c in APPEND_SINK_CASES])
def test_append_sink_parity(w, first, n, gpu_lib):
    say(f"case append+sink {w.name} first={first} n={n}")
    append_sink_case(w, first, n)


def test_append_sink_480p(gpu_lib):
    w = W.WAN13B_480P
    say(f"case append+sink {w.name}")
    append_sink_case(w, w.chunk_frames - 1, 1, rows=sample_rows(w.query_rows, 34, n_random=96))


@pytest.mark.parametrize("dtype,kv_splits", [("bf16", 0), ("fp32", 0), ("bf16", -1)])
def test_stream_with_refresh_and_sink_updates(dtype, kv_splits, gpu_lib):
    """A stream of 24 chunks from t0 = 0 with a RoPE refresh every 5 chunks
    and a sink update every 7, every chunk's output and the stamps checked
    against the oracle.  With kv_splits = -1 (balanced schedule) the sink
    slot holds a recent frame after an update, so the keys each chunk sees
    differ from the host's estimate of its work; the last segment of every
    query tile still covers the rest of its keys."""
    import torch

    from streaming_causal_video_amd import binding as B

    w = small(f"stream-rs-{dtype}", dtype=dtype, grid_h=4, grid_w=6, window_frames=5, seed=220)
    say(f"case streaming refresh/sink {w.name} kv_splits={kv_splits}")
    cache = B.Cache(B.config_for(w))
    sk = to_device(G.frames_tensor(w, G.TENSOR_K, [0], 1), dtype)
    sv = to_device(G.frames_tensor(w, G.TENSOR_V, [0], 1), dtype)
    cache.cache_init(sk, sv)
    oc = O.OracleCache(spec_of(w))
    oc.init(G.frames_tensor(w, G.TENSOR_K, [0], 1), G.frames_tensor(w, G.TENSOR_V, [0], 1))
    C = w.chunk_frames
    shape = (1, C * w.tokens_per_frame, w.heads, w.head_dim)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for step in range(24):
        t0 = [step * C]
        if step % 5 == 4:
            delta = [t0[0] - cache.time_offsets()[0] - 3]
            cache.rope_refresh(delta)
            oc.rope_refresh(delta)
        q = G.frames_tensor(w, G.TENSOR_Q, t0, C)
        k = G.frames_tensor(w, G.TENSOR_K, t0, C)
        v = G.frames_tensor(w, G.TENSOR_V, t0, C)
        q_rot = torch.empty(shape, dtype=tdt, device="cuda")
        o = torch.empty(shape, dtype=tdt, device="cuda")
        lse = torch.empty((1, w.heads, shape[1]), dtype=torch.float32, device="cuda")
        kd, vd = to_device(k, dtype), to_device(v, dtype)
        cache.rope3d_append(to_device(q, dtype), q_rot, kd, vd, t0, C)
        q_ref = oc.rope3d_append(q, k, v, t0, C)
        if step % 7 == 6:
            P = w.tokens_per_frame
            cache.sink_update(kd[:, :P].contiguous(), vd[:, :P].contiguous(), t0, 1)
            oc.sink_update(k[:, :P], v[:, :P], t0, 1)
        cache.chunk_attention(q_rot, t0, C, o, lse, kv_splits=kv_splits)
        torch.cuda.synchronize()
        O_ref, _ = oc.chunk_attention(q_ref, t0, C)
        check_values(f"step {step} o", to_np(o), O_ref, dtype)
        assert np.array_equal(cache.views()["stamps"].cpu().numpy(), oc.stamps)
        assert cache.time_offsets() == [int(x) for x in oc.pos_offset]
