"""The allocation-free chunk_attention (static scratch workspace) against the
entry point that takes a caller workspace: the same kernels under the same
forced schedule, so the outputs must agree bit for bit.  Two calls in a row,
the second on a smaller input; a schedule too large for the scratch fails
cleanly."""
import pytest

from parity_util import say
from streaming_causal_video_amd import binding as B
from streaming_causal_video_amd import workloads as W
from streaming_causal_video_amd.runner import StreamRunner

pytestmark = pytest.mark.gpu


def case(name, **kw):
    base = dict(
        name=name, dtype="bf16", batch=1, heads=2, head_dim=128, split=(44, 42, 42), base=10000.0, grid_h=4,
        grid_w=4, chunk_frames=2, sink_frames=1, window_frames=4, t0=(9,), seed=301,
    )
    base.update(kw)
    return W.Workload(**base)


# the larger call first, then a smaller one on a different cache
CALLS = [
    (case("scratch-big", batch=2, heads=4, grid_h=12, grid_w=20, chunk_frames=3, window_frames=6,
          max_query_chunks=2, t0=(40, 9), seed=302), -1),
    (case("scratch-small", grid_h=6, grid_w=10, t0=(17,), seed=303), 3),
]


def test_scratch_matches_workspace_entry(gpu_lib):
    import torch

    for w, kv in CALLS:
        say(f"case no-alloc {w.name} kv_splits={kv}")
        r = StreamRunner(w, kv_splits=kv)
        r.fill()
        r.append()
        need = r.cache.request_workspace_bytes(w.t0, r.n_frames, kv)
        assert 0 < need <= B.SCRATCH_BYTES, need
        r.attend()  # caller workspace (sized for this request)
        o_s = torch.empty_like(r.o)
        lse_s = torch.empty_like(r.lse)
        r.cache.chunk_attention_scratch(r.q_rot, w.t0, r.n_frames, o_s, lse_s, kv)
        torch.cuda.synchronize()
        assert torch.equal(o_s.view(torch.int16), r.o.view(torch.int16)), w.name
        assert torch.equal(lse_s.view(torch.int32), r.lse.view(torch.int32)), w.name


def test_scratch_rejects_oversize_schedule(gpu_lib):
    import torch

    w = W.WAN13B_480P
    r = StreamRunner(w, kv_splits=1, with_lse=False)
    r.fill()
    r.append()
    o = torch.zeros_like(r.o)
    with pytest.raises(B.ScvError) as ei:
        r.cache.chunk_attention_scratch(r.q_rot, w.t0, r.n_frames, o, None, 64)
    assert ei.value.status == -7
    torch.cuda.synchronize()
    assert int(o.abs().sum().item()) == 0  # nothing was enqueued
