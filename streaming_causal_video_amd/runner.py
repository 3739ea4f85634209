"""Drive the library over a workload: fill a cache, then run the step.

The step is the hot path of one attention layer for one query chunk:
``rope3d_append`` (rotate q, rotate k and append k, v into the ring) and
``chunk_attention``.  Inputs come from ``datagen`` (seeded synthetic values),
moved to the GPU once; everything after that runs in libscv's kernels.
"""
from __future__ import annotations

import numpy as np

from . import binding as B
from . import datagen as G
from .workloads import Workload, fill_schedule


def to_device(x: np.ndarray, dtype: str, device="cuda"):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)  # exact: the values are bf16-representable
    return t.to(device)


class StreamRunner:
    def __init__(self, w: Workload, kv_splits: int = 0, device="cuda", with_lse: bool = True):
        import torch

        self.w = w
        self.device = device
        self.cache = B.Cache(B.config_for(w), device=device)
        self.kv_splits = kv_splits
        nq = w.query_frames
        self.n_frames = nq
        shape = (w.batch, nq * w.tokens_per_frame, w.heads, w.head_dim)
        tdt = self.cache.dtype
        self.q = to_device(G.frames_tensor(w, G.TENSOR_Q, w.t0, nq), w.dtype, device)
        self.k = to_device(G.frames_tensor(w, G.TENSOR_K, w.t0, nq), w.dtype, device)
        self.v = to_device(G.frames_tensor(w, G.TENSOR_V, w.t0, nq), w.dtype, device)
        self.q_rot = torch.empty(shape, dtype=self.cache.qk_dtype, device=device)
        self.o = torch.empty(shape, dtype=tdt, device=device)
        self.lse = torch.empty((w.batch, w.heads, nq * w.tokens_per_frame), dtype=torch.float32, device=device) \
            if with_lse else None
        self.ws = self.cache.make_workspace(nq, kv_splits, t0=w.t0)
        ws_bytes = 0 if self.ws is None else self.ws.numel()
        self.splits = self.cache.attention_splits(nq, kv_splits, t0=w.t0, ws_bytes=ws_bytes)

    def fill(self, stream=None):
        """cache_init with the sink frames, then the window frames.  The
        input temporaries are allocated on torch's current stream; when the
        calls run on another `stream`, that use is recorded so that their
        memory is not reused before those kernels have read it."""
        w = self.w

        def used_on_stream(*ts):
            if stream is not None:
                for t in ts:
                    t.record_stream(stream)

        if w.sink_frames > 0:
            zeros = [0] * w.batch
            sk = to_device(G.frames_tensor(w, G.TENSOR_K, zeros, w.sink_frames), w.dtype, self.device)
            sv = to_device(G.frames_tensor(w, G.TENSOR_V, zeros, w.sink_frames), w.dtype, self.device)
            self.cache.cache_init(sk, sv, stream=stream)
            used_on_stream(sk, sv)
        else:
            self.cache.cache_init(stream=stream)
        for starts, n in fill_schedule(w):
            k = to_device(G.frames_tensor(w, G.TENSOR_K, starts, n), w.dtype, self.device)
            v = to_device(G.frames_tensor(w, G.TENSOR_V, starts, n), w.dtype, self.device)
            self.cache.rope3d_append(None, None, k, v, starts, n, stream=stream)
            used_on_stream(k, v)

    def append(self, stream=None):
        self.cache.rope3d_append(self.q, self.q_rot, self.k, self.v, self.w.t0, self.n_frames, stream=stream)

    def attend(self, stream=None):
        self.cache.chunk_attention(self.q_rot, self.w.t0, self.n_frames, self.o, self.lse, self.kv_splits, self.ws,
                                   stream=stream)

    def step(self, stream=None):
        self.append(stream)
        self.attend(stream)
