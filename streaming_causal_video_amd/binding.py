"""ctypes binding of libscv.so (declared in include/scv.h).

Argument marshalling only: torch tensors become device pointers, host int64
arrays become ``t0``, the current torch stream becomes the ``hipStream_t``.
Every step of the path runs in the library's HIP kernels; if the library is
missing this module raises instead of computing anything itself.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libscv.so")

SCV_FP32, SCV_BF16, SCV_FP16 = 0, 1, 2
SCRATCH_BYTES = 128 << 20  # SCV_SCRATCH_BYTES: the static workspace of scv_chunk_attention_scratch
_DTYPE_CODES = {"fp32": SCV_FP32, "bf16": SCV_BF16, "fp16": SCV_FP16}
STATUS_NAMES = {
    0: "SCV_OK",
    -1: "SCV_E_INVALID",
    -2: "SCV_E_SHAPE",
    -3: "SCV_E_DTYPE",
    -4: "SCV_E_ALIGN",
    -5: "SCV_E_RANGE",
    -6: "SCV_E_STATE",
    -7: "SCV_E_WORKSPACE",
    -8: "SCV_E_HIP",
}


class ScvConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rope_split", ctypes.c_int32 * 3),
        ("rope_base", ctypes.c_double),
        ("grid_h", ctypes.c_int32),
        ("grid_w", ctypes.c_int32),
        ("sink_frames", ctypes.c_int32),
        ("window_frames", ctypes.c_int32),
        ("chunk_frames", ctypes.c_int32),
        ("max_query_chunks", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("qk_dtype", ctypes.c_int32),
    ]


class ScvLayout(ctypes.Structure):
    _fields_ = [
        ("total_bytes", ctypes.c_size_t),
        ("stamps_offset", ctypes.c_size_t),
        ("table_h_offset", ctypes.c_size_t),
        ("table_w_offset", ctypes.c_size_t),
        ("k_offset", ctypes.c_size_t),
        ("v_offset", ctypes.c_size_t),
        ("n_slots", ctypes.c_int64),
        ("ring_frames", ctypes.c_int64),
        ("slot_rows", ctypes.c_int64),
        ("rows", ctypes.c_int64),
        ("rows_pad", ctypes.c_int64),
        ("elem_bytes", ctypes.c_int64),
    ]


class ScvError(RuntimeError):
    def __init__(self, status: int, what: str, msg: str):
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None

_VP, _I64P, _FP = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_float)
_SIGNATURES = {
    "scv_cache_bytes": (ctypes.c_size_t, [ctypes.POINTER(ScvConfig)]),
    "scv_cache_layout_of": (ctypes.c_int, [ctypes.POINTER(ScvConfig), ctypes.POINTER(ScvLayout)]),
    "scv_cache_create": (ctypes.c_int, [ctypes.POINTER(ScvConfig), _VP, ctypes.c_size_t, ctypes.POINTER(_VP)]),
    "scv_cache_destroy": (ctypes.c_int, [_VP]),
    "scv_cache_init": (ctypes.c_int, [_VP, _VP, _VP, _VP]),
    "scv_rope3d_apply": (ctypes.c_int, [_VP, _VP, _VP, _I64P, ctypes.c_int32, _VP]),
    "scv_kv_append_roll": (ctypes.c_int, [_VP, _VP, _VP, _I64P, ctypes.c_int32, _VP]),
    "scv_rope3d_append": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _I64P, ctypes.c_int32, _VP]),
    "scv_qkv_rope_append": (ctypes.c_int, [_VP, _VP, ctypes.c_int32, _VP, _VP, _I64P, ctypes.c_int32, _VP]),
    "scv_rope_refresh": (ctypes.c_int, [_VP, _I64P, _VP]),
    "scv_time_offsets": (ctypes.c_int, [_VP, _I64P]),
    "scv_sink_update": (ctypes.c_int, [_VP, _VP, _VP, _I64P, ctypes.c_int32, _VP]),
    "scv_rope3d_append_sink": (
        ctypes.c_int,
        [_VP, _VP, _VP, _VP, _VP, _I64P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _VP],
    ),
    "scv_attention_splits": (ctypes.c_int32, [_VP, _I64P, ctypes.c_int32, ctypes.c_int32, ctypes.c_size_t]),
    "scv_attention_workspace_bytes": (ctypes.c_size_t, [_VP, ctypes.c_int32, ctypes.c_int32]),
    "scv_attention_request_workspace_bytes": (ctypes.c_size_t, [_VP, _I64P, ctypes.c_int32, ctypes.c_int32]),
    "scv_chunk_attention": (
        ctypes.c_int,
        [_VP, _VP, _I64P, ctypes.c_int32, _VP, _VP, ctypes.c_int32, _VP, ctypes.c_size_t, _VP],
    ),
    "scv_chunk_attention_scratch": (
        ctypes.c_int,
        [_VP, _VP, _I64P, ctypes.c_int32, _VP, _VP, ctypes.c_int32, _VP],
    ),
    "scv_rope_table_floats": (ctypes.c_size_t, [_VP, ctypes.c_int32]),
    "scv_rope_tables": (ctypes.c_int, [_VP, _I64P, ctypes.c_int32, _VP, ctypes.c_size_t, _VP]),
    "scv_debug_stamps": (ctypes.c_int, [_VP, _I64P, ctypes.c_size_t]),
    "scv_last_error": (ctypes.c_char_p, []),
}


def load(path: str = LIB_PATH):
    """Load libscv.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def last_error() -> str:
    return load().scv_last_error().decode(errors="replace")


def _check(status: int, what: str):
    if status != 0:
        raise ScvError(status, what, last_error())


def make_config(
    *,
    batch,
    heads,
    head_dim,
    split,
    base,
    grid_h,
    grid_w,
    sink_frames,
    window_frames,
    chunk_frames,
    max_query_chunks=1,
    dtype="bf16",
    qk_dtype="",
) -> ScvConfig:
    c = ScvConfig()
    c.batch, c.heads, c.head_dim = batch, heads, head_dim
    c.rope_split[0], c.rope_split[1], c.rope_split[2] = split
    c.rope_base = float(base)
    c.grid_h, c.grid_w = grid_h, grid_w
    c.sink_frames, c.window_frames, c.chunk_frames = sink_frames, window_frames, chunk_frames
    c.max_query_chunks = max_query_chunks
    c.dtype = _DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)
    c.qk_dtype = (_DTYPE_CODES[qk_dtype] if qk_dtype else 0) if isinstance(qk_dtype, str) else int(qk_dtype)
    return c


def config_for(w) -> ScvConfig:
    """Config of a ``workloads.Workload``."""
    return make_config(
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
        dtype=w.dtype,
        qk_dtype=w.qk_dtype,
    )


def cache_bytes(cfg: ScvConfig) -> int:
    return int(load().scv_cache_bytes(ctypes.byref(cfg)))


def cache_layout(cfg: ScvConfig) -> ScvLayout:
    L = ScvLayout()
    _check(load().scv_cache_layout_of(ctypes.byref(cfg), ctypes.byref(L)), "scv_cache_layout_of")
    return L


def _t0_array(t0: Sequence[int], batch: int):
    vals = [int(x) for x in t0]
    if len(vals) != batch:
        raise ValueError(f"t0 has {len(vals)} entries, batch is {batch}")
    return (ctypes.c_int64 * batch)(*vals)


def _ptr(x) -> Optional[int]:
    return None if x is None else x.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class Cache:
    """A streaming KV cache: a caller-owned device buffer plus its handle."""

    def __init__(self, cfg: ScvConfig, device="cuda"):
        import torch

        self.cfg = cfg
        self.lib = load()
        self.layout = cache_layout(cfg)
        self.nbytes = int(self.layout.total_bytes)
        self.buffer = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        tmap = {SCV_FP32: torch.float32, SCV_BF16: torch.bfloat16, SCV_FP16: torch.float16}
        self.dtype = tmap[cfg.dtype]
        self.qk_dtype = tmap[cfg.qk_dtype or cfg.dtype]
        self.P = cfg.grid_h * cfg.grid_w
        h = _VP()
        _check(self.lib.scv_cache_create(ctypes.byref(cfg), self.buffer.data_ptr(), self.nbytes, ctypes.byref(h)),
               "scv_cache_create")
        self.handle = h

    # -- tensor checks (marshalling) ------------------------------------
    def _tok(self, x, n_frames, name, rotated=False):
        if x is None:
            return None
        c = self.cfg
        want = (c.batch, n_frames * self.P, c.heads, c.head_dim)
        dt = self.qk_dtype if rotated else self.dtype
        if tuple(x.shape) != want or x.dtype != dt or not x.is_cuda or not x.is_contiguous():
            raise ValueError(f"{name}: need contiguous {dt} cuda tensor {want}, got {x.dtype} {tuple(x.shape)}")
        return x

    # -- the four calls ---------------------------------------------------
    def cache_init(self, sink_k=None, sink_v=None, stream=None):
        sf = self.cfg.sink_frames
        self._tok(sink_k, sf, "sink_k")
        self._tok(sink_v, sf, "sink_v")
        _check(self.lib.scv_cache_init(self.handle, _ptr(sink_k), _ptr(sink_v), _stream(stream)), "scv_cache_init")

    def rope3d_apply(self, q, k, t0, n_frames, stream=None):
        """Rotates q and/or k in place; returns them viewed in the rotated
        (qk) dtype, which is what their buffers hold afterwards."""
        self._tok(q, n_frames, "q")
        self._tok(k, n_frames, "k")
        _check(
            self.lib.scv_rope3d_apply(self.handle, _ptr(q), _ptr(k), _t0_array(t0, self.cfg.batch), n_frames,
                                      _stream(stream)),
            "scv_rope3d_apply",
        )
        return (None if q is None else q.view(self.qk_dtype), None if k is None else k.view(self.qk_dtype))

    def kv_append_roll(self, k_rot, v, t0, n_frames, stream=None):
        self._tok(k_rot, n_frames, "k_rot", rotated=True)
        self._tok(v, n_frames, "v")
        _check(
            self.lib.scv_kv_append_roll(self.handle, _ptr(k_rot), _ptr(v), _t0_array(t0, self.cfg.batch), n_frames,
                                        _stream(stream)),
            "scv_kv_append_roll",
        )

    def rope3d_append(self, q, q_rot, k, v, t0, n_frames, stream=None):
        self._tok(q, n_frames, "q")
        self._tok(q_rot, n_frames, "q_rot", rotated=True)
        self._tok(k, n_frames, "k")
        self._tok(v, n_frames, "v")
        _check(
            self.lib.scv_rope3d_append(self.handle, _ptr(q), _ptr(q_rot), _ptr(k), _ptr(v),
                                       _t0_array(t0, self.cfg.batch), n_frames, _stream(stream)),
            "scv_rope3d_append",
        )

    def qkv_rope_append(self, x, w_qkv, q_rot, t0, n_frames, stream=None):
        """Projection of the layer input x [B, n*P, d_model] by w_qkv
        [3*H*d, d_model], with RoPE and the cache append fused in."""
        c = self.cfg
        d_model = int(x.shape[-1]) if x is not None else 0
        want_x = (c.batch, n_frames * self.P, d_model)
        if x is None or tuple(x.shape) != want_x or x.dtype != self.dtype or not x.is_contiguous():
            raise ValueError(f"x: need contiguous {self.dtype} tensor {want_x}")
        want_w = (3 * c.heads * c.head_dim, d_model)
        if w_qkv is None or tuple(w_qkv.shape) != want_w or w_qkv.dtype != self.dtype or not w_qkv.is_contiguous():
            raise ValueError(f"w_qkv: need contiguous {self.dtype} tensor {want_w}")
        self._tok(q_rot, n_frames, "q_rot", rotated=True)
        _check(
            self.lib.scv_qkv_rope_append(self.handle, _ptr(x), d_model, _ptr(w_qkv), _ptr(q_rot),
                                         _t0_array(t0, c.batch), n_frames, _stream(stream)),
            "scv_qkv_rope_append",
        )

    def rope_refresh(self, delta, stream=None):
        """Move each stream's time origin forward by delta[b] frames (cached
        keys re-rotated on the device)."""
        _check(self.lib.scv_rope_refresh(self.handle, _t0_array(delta, self.cfg.batch), _stream(stream)),
               "scv_rope_refresh")

    def time_offsets(self):
        out = (ctypes.c_int64 * self.cfg.batch)()
        _check(self.lib.scv_time_offsets(self.handle, out), "scv_time_offsets")
        return [int(x) for x in out]

    def sink_update(self, k, v, first_frame, n_frames, stream=None):
        """Sink slots 0..n_frames-1 take frames first_frame[b] + j (raw k, v)."""
        self._tok(k, n_frames, "k")
        self._tok(v, n_frames, "v")
        _check(
            self.lib.scv_sink_update(self.handle, _ptr(k), _ptr(v), _t0_array(first_frame, self.cfg.batch), n_frames,
                                     _stream(stream)),
            "scv_sink_update",
        )

    def rope3d_append_sink(self, q, q_rot, k, v, t0, n_frames, sink_first, sink_frames, stream=None):
        """rope3d_append, and frames sink_first .. sink_first+sink_frames-1 of
        the same k, v also written into sink slots 0 .. sink_frames-1."""
        self._tok(q, n_frames, "q")
        self._tok(q_rot, n_frames, "q_rot", rotated=True)
        self._tok(k, n_frames, "k")
        self._tok(v, n_frames, "v")
        _check(
            self.lib.scv_rope3d_append_sink(self.handle, _ptr(q), _ptr(q_rot), _ptr(k), _ptr(v),
                                            _t0_array(t0, self.cfg.batch), n_frames, int(sink_first),
                                            int(sink_frames), _stream(stream)),
            "scv_rope3d_append_sink",
        )

    SCHEDULE_BALANCED = -1
    SCHEDULE_ROUNDS = -2

    def attention_splits(self, n_frames, kv_splits=0, t0=None, ws_bytes=None) -> int:
        """Schedule chunk_attention uses: a split count, or -1 for the
        balanced schedule (t0: the request's start frames or None for the
        steady-state estimate; ws_bytes: the workspace it will get)."""
        t = None if t0 is None else _t0_array(t0, self.cfg.batch)
        lim = (1 << 64) - 1 if ws_bytes is None else int(ws_bytes)
        return int(self.lib.scv_attention_splits(self.handle, t, n_frames, kv_splits, lim))

    def workspace_bytes(self, n_frames, kv_splits=0) -> int:
        return int(self.lib.scv_attention_workspace_bytes(self.handle, n_frames, kv_splits))

    def request_workspace_bytes(self, t0, n_frames, kv_splits=0) -> int:
        """Workspace of the schedule this request (its t0) selects."""
        return int(self.lib.scv_attention_request_workspace_bytes(self.handle, _t0_array(t0, self.cfg.batch),
                                                                  n_frames, kv_splits))

    def make_workspace(self, n_frames, kv_splits=0, t0=None):
        import torch

        n = self.workspace_bytes(n_frames, kv_splits) if t0 is None else \
            self.request_workspace_bytes(t0, n_frames, kv_splits)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.buffer.device) if n else None

    def chunk_attention(self, q_rot, t0, n_frames, o, lse=None, kv_splits=0, ws=None, stream=None):
        import torch

        self._tok(q_rot, n_frames, "q_rot", rotated=True)
        self._tok(o, n_frames, "o")
        if lse is not None:
            want = (self.cfg.batch, self.cfg.heads, n_frames * self.P)
            if tuple(lse.shape) != want or lse.dtype != torch.float32 or not lse.is_contiguous():
                raise ValueError(f"lse: need contiguous float32 {want}")
        if ws is None:
            # the schedule this request gets (from its t0), then exactly its
            # workspace (None when it runs unsplit).  The workspace comes from
            # torch's allocator on its current stream but is used on
            # `stream`: record that use so the block is not handed out again
            # before the kernels on `stream` are done with it.
            kv_splits = self.attention_splits(n_frames, kv_splits, t0=t0)
            ws = self.make_workspace(n_frames, kv_splits, t0=t0)
            if ws is not None and stream is not None:
                ws.record_stream(stream)
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
        _check(
            self.lib.scv_chunk_attention(self.handle, _ptr(q_rot), _t0_array(t0, self.cfg.batch), n_frames, _ptr(o),
                                         _ptr(lse), kv_splits, _ptr(ws), ws_bytes, _stream(stream)),
            "scv_chunk_attention",
        )

    def chunk_attention_scratch(self, q_rot, t0, n_frames, o, lse=None, kv_splits=0, stream=None):
        """chunk_attention with the library's static scratch as workspace:
        allocates nothing (calls overlapping on one GPU race)."""
        import torch

        self._tok(q_rot, n_frames, "q_rot", rotated=True)
        self._tok(o, n_frames, "o")
        if lse is not None:
            want = (self.cfg.batch, self.cfg.heads, n_frames * self.P)
            if tuple(lse.shape) != want or lse.dtype != torch.float32 or not lse.is_contiguous():
                raise ValueError(f"lse: need contiguous float32 {want}")
        _check(
            self.lib.scv_chunk_attention_scratch(self.handle, _ptr(q_rot), _t0_array(t0, self.cfg.batch), n_frames,
                                                 _ptr(o), _ptr(lse), kv_splits, _stream(stream)),
            "scv_chunk_attention_scratch",
        )

    def rope_tables(self, t0, n_frames, stream=None):
        """fp32 tables as the kernels compute them: dict t [B,n,dt/2,2],
        h [grid_h,dh/2,2], w [grid_w,dw/2,2] (device tensors)."""
        import torch

        c = self.cfg
        n = int(self.lib.scv_rope_table_floats(self.handle, n_frames))
        out = torch.empty(n, dtype=torch.float32, device=self.buffer.device)
        _check(
            self.lib.scv_rope_tables(self.handle, _t0_array(t0, c.batch), n_frames, out.data_ptr(), n,
                                     _stream(stream)),
            "scv_rope_tables",
        )
        dt, dh, dw = c.rope_split
        nt = c.batch * n_frames * (dt // 2) * 2
        nh = c.grid_h * (dh // 2) * 2
        return {
            "t": out[:nt].view(c.batch, n_frames, dt // 2, 2),
            "h": out[nt : nt + nh].view(c.grid_h, dh // 2, 2),
            "w": out[nt + nh :].view(c.grid_w, dw // 2, 2),
        }

    def debug_stamps(self):
        """Slot stamps [B][n_slots] copied to the host by the library (the
        call synchronises the device)."""
        c = self.cfg
        n = c.batch * int(self.layout.n_slots)
        out = (ctypes.c_int64 * n)()
        _check(self.lib.scv_debug_stamps(self.handle, out, n), "scv_debug_stamps")
        return [[int(out[b * int(self.layout.n_slots) + s]) for s in range(int(self.layout.n_slots))]
                for b in range(c.batch)]

    def views(self):
        """Typed views of the cache buffer, per the documented layout."""
        import torch

        c, L, buf = self.cfg, self.layout, self.buffer
        eb = int(L.elem_bytes)
        kv = c.batch * c.heads * int(L.rows_pad) * c.head_dim * eb
        dt, dh, dw = c.rope_split
        return {
            "stamps": buf[L.stamps_offset : L.stamps_offset + c.batch * L.n_slots * 8].view(torch.int64).view(
                c.batch, int(L.n_slots)),
            "table_h": buf[L.table_h_offset : L.table_h_offset + c.grid_h * (dh // 2) * 8].view(torch.float32).view(
                c.grid_h, dh // 2, 2),
            "table_w": buf[L.table_w_offset : L.table_w_offset + c.grid_w * (dw // 2) * 8].view(torch.float32).view(
                c.grid_w, dw // 2, 2),
            "k": buf[L.k_offset : L.k_offset + kv].view(self.qk_dtype).view(c.batch, c.heads, int(L.rows_pad),
                                                                             c.head_dim),
            "v_t": buf[L.v_offset : L.v_offset + kv].view(self.dtype).view(c.batch, c.heads, c.head_dim,
                                                                            int(L.rows_pad)),
        }

    def close(self):
        if getattr(self, "handle", None):
            self.lib.scv_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
