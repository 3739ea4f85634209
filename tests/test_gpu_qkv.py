"""GPU parity of the fused QKV projection + 3D RoPE + append (through the C
ABI) against the fp64 oracle (projection, then rope3d_append).

Bars: relative L2 <= 1e-2 for q_rot, the cached keys and values and the
attention output over the cache the fused call filled; stamps bit-exact.
Element-wise, every output is within one rounding of the storage dtype plus
the fp32 accumulation error of the projection (1e-4 of the tensor's rms).
"""
import numpy as np
import pytest

from parity_util import check_values, oracle_fill, sample_rows, say, to_np
from streaming_causal_video_amd import datagen as G
from streaming_causal_video_amd import workloads as W
from streaming_causal_video_amd.runner import StreamRunner, to_device

pytestmark = pytest.mark.gpu


def small(name, d_model, **kw):
    base = dict(
        name=name, dtype="bf16", batch=1, heads=2, head_dim=128, split=(44, 42, 42), base=10000.0, grid_h=4,
        grid_w=6, chunk_frames=2, sink_frames=1, window_frames=4, t0=(9,), seed=301,
    )
    base.update(kw)
    return W.Workload(**base), d_model


CASES = [
    small("qkv-d128", 64),
    small("qkv-d128-dm256-b2", 256, batch=2, heads=3, grid_h=6, grid_w=10, chunk_frames=3, window_frames=5,
          t0=(40, 3), seed=302),
    small("qkv-d64-dm96", 96, heads=4, head_dim=64, split=(24, 20, 20), grid_h=5, grid_w=8, sink_frames=2,
          window_frames=3, t0=(11,), seed=303),
    small("qkv-odd-grid", 128, grid_h=3, grid_w=5, window_frames=3, t0=(7,), seed=304),  # P = 15: V tail path
    small("qkv-qkfp16", 160, grid_h=6, grid_w=8, t0=(3000,), qk_dtype="fp16", seed=305),
    small("qkv-long-tiles", 192, heads=2, grid_h=20, grid_w=26, chunk_frames=2, window_frames=6, t0=(50,), seed=306),
    small("qkv-t0-0", 64, batch=2, t0=(0, 1), seed=307),
    small("qkv-multichunk", 96, grid_h=5, grid_w=12, window_frames=3, max_query_chunks=3, t0=(20,), seed=308),
]


def qk(w):
    return w.qk_dtype or w.dtype


def close_elementwise(name, got, ref, dtype):
    rel = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}[dtype]
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bad = np.abs(got - ref) > rel * np.abs(ref) + 1e-4 * rms
    assert not bad.any(), (name, int(bad.sum()), float(np.max(np.abs(got - ref))))


def run_case(w, d_model, rows=None, heads=None, refresh=0):
    import torch

    r = StreamRunner(w)
    r.fill()
    oc = oracle_fill(w)
    if refresh:
        delta = [refresh] * w.batch
        r.cache.rope_refresh(delta)
        oc.rope_refresh(delta)
    n = w.query_frames
    x = G.hidden_frames(w, d_model, w.t0, n)
    wq = G.qkv_weight(w, d_model)
    xd = to_device(x, "bf16")
    wd = to_device(wq, "bf16")
    r.cache.qkv_rope_append(xd, wd, r.q_rot, w.t0, n)
    r.attend()
    torch.cuda.synchronize()
    q_ref = oc.qkv_rope_append(x, wq, w.t0, n)
    qg = to_np(r.q_rot)
    check_values("q_rot", qg, q_ref, "bf16", per_axis0=True)
    close_elementwise("q_rot", qg, q_ref, qk(w))
    v = r.cache.views()
    assert np.array_equal(v["stamps"].cpu().numpy(), oc.stamps)
    L = r.cache.layout
    P = w.tokens_per_frame
    hs = list(range(w.heads)) if heads is None else heads
    for b in range(w.batch):
        for f in range(n):
            s = int(np.nonzero(oc.stamps[b] == w.t0[b] + f)[0][0])
            rws = slice(s * L.slot_rows, s * L.slot_rows + P)
            kg = to_np(v["k"][b, hs, rws, :]).transpose(1, 0, 2)
            vg = to_np(v["v_t"][b, hs, :, rws]).transpose(2, 0, 1)
            kr, vr = oc.k[b][s][:, hs], oc.v[b][s][:, hs]
            check_values(f"k frame {f}", kg, kr, "bf16")
            check_values(f"v frame {f}", vg, vr, "bf16")
            close_elementwise("k", kg, kr, qk(w))
            close_elementwise("v", vg, vr, "bf16")
    O_ref, _ = oc.chunk_attention(q_ref, w.t0, n, rows=rows)
    o = to_np(r.o)
    if rows is not None:
        o = o[:, rows]
    check_values("o", o, O_ref, "bf16", per_axis0=True)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0].name)
def test_qkv_rope_append_parity(case, gpu_lib):
    w, d_model = case
    say(f"case qkv {w.name} d_model={d_model}")
    run_case(w, d_model)


def test_qkv_after_refresh(gpu_lib):
    w, d_model = CASES[1]
    say(f"case qkv-refresh {w.name}")
    run_case(w, d_model, refresh=3)


def test_qkv_480p(gpu_lib):
    w = W.WAN13B_480P
    say(f"case qkv {w.name} d_model=1536")
    run_case(w, 1536, rows=sample_rows(w.query_rows, 41, n_random=64), heads=[0, 5, w.heads - 1])
