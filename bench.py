"""Benchmark of the streaming chunk-attention hot path on one GPU.

A step is one pass of the whole path for one query chunk of one attention
layer: rope3d_append (3D RoPE of q and k at the global time index, append
of k/v into the sink-pinned ring) followed by chunk_attention over sink +
window + chunk.  Inputs are seeded synthetic tensors already resident in
HBM; the cache is filled before the timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line (rank 0).  The dominant kernel's roofline comes from
HIP events recorded around its launches inside the timed region, on the
stream the kernels run on; cpu_baseline times the fp64 oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense bf16 MFMA peak: 256 CUs x 2.4 GHz x 4096 flop/clk/CU (the
# published 2.5 PFLOP/s); fp32 MFMA/vector 157.3 TFLOP/s.
PEAK_TFLOPS = {"bf16": 2516.6, "fp32": 157.3}
HBM_PEAK_GBS = 8000.0

# HBM bytes per launch of the attention kernel, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE counter runs scaled by the same counters on a plain copy of
# known size (bench.py --calibrate-copy).  Valid only for the kernel source
# they were taken on: any other source hash reports null.
MEASURED_TRAFFIC = {
    # profiles/chunk_attn_wan13b_480p.md (grid schedule, one launch)
    "wan1.3b-480p": {"source": "39c1999d5fe07a07", "kv_splits": 1, "bytes_per_launch": 380914995},
    # profiles/chunk_attn_wan13b_720p_balanced.md (balanced schedule with
    # whole-item rounds: the attention launch and its merge launch, as timed
    # together)
    "wan1.3b-720p": {"source": "39c1999d5fe07a07", "kv_splits": -2, "bytes_per_launch": 972712435},
}
KERNEL_SOURCES = [
    "streaming_causal_video_amd/csrc/chunk_attn.hip",
    "streaming_causal_video_amd/csrc/scv_internal.h",
    "streaming_causal_video_amd/csrc/scv_abi.cpp",  # the schedule the host picks
]


def kernel_source_hash():
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def calibrate_copy(nbytes):
    """A plain device-to-device copy of nbytes (read nbytes, write nbytes),
    repeated 5 times: the reference for scaling the HBM byte counters."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "launches": 5}), flush=True)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_pairs(w, stamps):
    """Query-key pairs the block-causal sink + window rule admits, per
    stream, from the slot stamps the cache holds after the step's append."""
    P, C = w.tokens_per_frame, w.chunk_frames
    total = 0
    for b in range(w.batch):
        for c in range((w.query_frames + C - 1) // C):
            s = w.t0[b] + c * C
            rows = min(C, w.query_frames - c * C) * P
            frames = 0
            for g in stamps[b]:
                g = int(g)
                if g >= 0 and g < s + C and (g < w.sink_frames or g >= s - w.window_frames):
                    frames += 1
            total += rows * frames * P
    return total


def _host_info():
    """Host CPU model, logical CPU count and the BLAS thread count numpy uses."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info

        blas = max([int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "blas_threads": blas}


def cpu_baseline(w, budget_s=20.0):
    """The fp64 oracle (as it stands) on the same workload, timed on the host
    cores: its rope3d_append of the query chunk (whole chunk) plus its chunk
    attention on a random sample of query rows (all heads, all visible keys)
    scaled to every row; each part the median of 3 runs.  Returns TFLOP/s of
    that step (attention FLOPs per step time) and latent frames/s."""
    import numpy as np

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity_util import oracle_fill

    from streaming_causal_video_amd import datagen as G

    info = _host_info()
    log("cpu_baseline: oracle fill (untimed) ...")
    oc = oracle_fill(w)
    nq = w.query_frames
    q = G.frames_tensor(w, G.TENSOR_Q, w.t0, nq)
    k = G.frames_tensor(w, G.TENSOR_K, w.t0, nq)
    v = G.frames_tensor(w, G.TENSOR_V, w.t0, nq)

    def median3(fn):
        ts = []
        for _ in range(3):
            t = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t)
        return sorted(ts)[1]

    holder = {}
    t_ra = median3(lambda: holder.__setitem__("q_rot", oc.rope3d_append(q, k, v, w.t0, nq)))
    q_rot = holder["q_rot"]
    rng = np.random.default_rng(0)
    # calibrate the row sample so that one attention run takes ~budget/6
    t = time.perf_counter()
    oc.chunk_attention(q_rot, w.t0, nq, rows=np.sort(rng.choice(w.query_rows, 32, replace=False)))
    per_row = (time.perf_counter() - t) / 32
    n = int(min(w.query_rows, max(32, (budget_s / 6.0 - 3 * t_ra / 6.0) / max(per_row, 1e-6))))
    rows = np.sort(rng.choice(w.query_rows, n, replace=False))
    t_att = median3(lambda: oc.chunk_attention(q_rot, w.t0, nq, rows=rows)) * (w.query_rows / n)
    keys = sum(len(oc.visible_slots(b, w.t0[b])) for b in range(w.batch)) * w.tokens_per_frame
    flops = 4 * w.head_dim * w.heads * w.query_rows * keys
    step_s = t_ra + t_att
    return {
        "value": flops / step_s / 1e12,
        "unit": "TFLOP/s",
        "cores": info["blas_threads"] or info["cpu_count"],
        "kind": "oracle",
        "sample": f"fp64 numpy oracle on {w.name}: rope3d_append of the whole query chunk ({t_ra:.2f} s) plus chunk "
        f"attention of {n} random query rows (all {w.heads} heads, all visible keys) scaled to {w.query_rows} rows "
        f"({t_att:.1f} s); each part the median of 3 runs; cache filled by the oracle beforehand (untimed)",
        "latent_frames_per_s": w.batch * w.query_frames / step_s,
        "step_s": step_s,
        **info,
    }


SAMPLER = r"""
import json, subprocess, sys, time
out, stop, exe = sys.argv[1], sys.argv[2], sys.argv[3]
t_end = time.time() + 600
with open(out, "w") as f:
    while time.time() < t_end:
        try:
            open(stop).close()
            break
        except OSError:
            pass
        t = time.time()
        try:
            p = subprocess.run([exe, "metric", "--clock", "--json"], capture_output=True, text=True, timeout=20)
            f.write(json.dumps({"t0": t, "t1": time.time(), "out": p.stdout}) + "\n")
            f.flush()
        except Exception:
            pass
        time.sleep(0.1)
"""


def start_clock_sampler():
    """Starts, before this process touches the GPU, a child process that
    polls amd-smi's per-XCD shader clock with wall-clock timestamps (the
    bench itself never starts a program after it has initialised the GPU).
    Returns a handle for read_clock_samples, or None without amd-smi."""
    import shutil
    import subprocess
    import tempfile

    exe = shutil.which("amd-smi") or ("/opt/rocm/bin/amd-smi" if os.path.exists("/opt/rocm/bin/amd-smi") else None)
    if exe is None:
        return None
    d = tempfile.mkdtemp(prefix="scv_clk_")
    out, stop = os.path.join(d, "samples.jsonl"), os.path.join(d, "stop")
    proc = subprocess.Popen([sys.executable, "-c", SAMPLER, out, stop, exe], stdout=subprocess.DEVNULL,
                            stderr=subprocess.DEVNULL)
    import atexit

    atexit.register(lambda: open(stop, "w").close())  # the sampler ends with the bench, whatever happens
    return {"proc": proc, "out": out, "stop": stop}


def read_clock_samples(h, t_lo, t_hi):
    """Stops the sampler; mean per-XCD shader clock (MHz) over the samples
    taken entirely inside the wall-clock window [t_lo, t_hi]."""
    if h is None:
        return None
    open(h["stop"], "w").close()
    try:
        h["proc"].wait(timeout=30)
    except Exception:  # pragma: no cover
        h["proc"].kill()
    clocks, n = [], 0
    try:
        lines = open(h["out"]).read().splitlines()
    except OSError:
        return None
    for line in lines:
        rec = json.loads(line)
        if rec["t0"] < t_lo or rec["t1"] > t_hi:
            continue
        try:
            data = json.loads(rec["out"])
        except ValueError:
            continue
        n += 1
        for gpu in data.get("gpu_data", []):
            for key, val in gpu.get("clock", {}).items():
                if key.lower().startswith("gfx_") and isinstance(val, dict):
                    c = val.get("clk", {})
                    c = c.get("value") if isinstance(c, dict) else c
                    try:
                        clocks.append(float(c))
                    except (TypeError, ValueError):
                        pass
    if not clocks:
        return None
    return {"mhz_mean": sum(clocks) / len(clocks), "mhz_min": min(clocks), "mhz_max": max(clocks), "samples": n,
            "source": "amd-smi metric --clock (per XCD), polled by a helper process while attention launches ran "
            "back to back for 3 s after the timed steps"}


def load_window(r, seconds=3.0):
    """Back-to-back attention launches for `seconds` (wall clock); returns
    the window and the mean time per launch over it (HIP events on the
    launch stream around all of its launches)."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 0
    t_lo = time.time()
    e0.record()
    while time.time() < t_lo + seconds:
        for _ in range(100):
            r.attend()
        n += 100
        torch.cuda.synchronize()
    e1.record()
    torch.cuda.synchronize()
    return (t_lo + 0.5, time.time()), {"ms": e0.elapsed_time(e1) / n, "launches": n}


def cold_step_ms(r, reps=5, flush_bytes=512 << 20):
    """Mean append and attention times with L2 and the 256 MB Infinity Cache
    flushed before each step by a 512 MB device write (outside the events)."""
    import torch

    junk = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    app = att = 0.0
    for _ in range(reps):
        junk.fill_(1)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        r.append()
        e[1].record()
        r.attend()
        e[2].record()
        torch.cuda.synchronize()
        app += e[0].elapsed_time(e[1])
        att += e[1].elapsed_time(e[2])
    del junk
    return {"append_ms": app / reps, "attn_ms": att / reps, "reps": reps, "flush_bytes": flush_bytes}


def ablations(w):
    """Before/after timings of design choices that can be switched from the
    API: fused rope3d_append vs rope3d_apply + kv_append_roll, and every
    attention schedule (key splits 1/2/4/8, balanced, whole-item rounds)
    against the host model's own choice.  One JSON line."""
    import torch

    from streaming_causal_video_amd.runner import StreamRunner

    def timed(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / reps

    out = {"workload": w.name}
    r = StreamRunner(w, kv_splits=1)
    r.fill()
    r.step()
    torch.cuda.synchronize()
    q_tmp, k_tmp = r.q.clone(), r.k.clone()

    def unfused():
        q_tmp.copy_(r.q)
        k_tmp.copy_(r.k)
        r.cache.rope3d_apply(q_tmp, k_tmp, w.t0, r.n_frames)
        r.cache.kv_append_roll(k_tmp.view(r.cache.qk_dtype), r.v, w.t0, r.n_frames)

    def copies():
        q_tmp.copy_(r.q)
        k_tmp.copy_(r.k)

    out["append_fused_ms"] = timed(r.append)
    out["append_unfused_ms"] = timed(unfused) - timed(copies)
    # every schedule the host can pick, the one its model picks for this
    # request (kv_splits = 0), and how far that one is from the fastest
    names = {-2: "rounds", -1: "balanced"}
    sched = {}
    for sp in (1, 2, 4, 8, -1, -2):
        rs = StreamRunner(w, kv_splits=sp)
        if rs.splits != sp:  # falls back where the schedule does not apply
            continue
        rs.fill()
        rs.step()
        sched[names.get(sp, f"splits_{sp}")] = timed(rs.attend)
        del rs
    auto = StreamRunner(w, kv_splits=0).splits
    auto_name = names.get(auto, f"splits_{auto}")
    if auto_name not in sched:
        ra = StreamRunner(w, kv_splits=auto)
        ra.fill()
        ra.step()
        sched[auto_name] = timed(ra.attend)
    best = min(sched, key=sched.get)
    out["attn_ms_by_schedule"] = sched
    out["model_choice"] = auto_name
    out["fastest"] = best
    out["model_choice_vs_fastest"] = sched[auto_name] / sched[best] - 1.0
    print(json.dumps(out), flush=True)


def back_to_back_us(fn, reps):
    """Mean time per launch of reps back-to-back launches of fn, from one
    pair of HIP events on the launch stream around all of them (a pair
    around each launch would add the launch latency of an idle queue to
    every one: ~10 us on a 80 us projection)."""
    import torch

    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / reps


def time_qkv(r, w, reps=20):
    """HIP-event time of the QKV projection fused with RoPE and the append
    (d_model = heads * head_dim, the Wan layers' width), replacing the
    step's rope3d_append: FLOPs 2 * tokens * d_model * 3*H*d."""
    from streaming_causal_video_amd import datagen as G
    from streaming_causal_video_amd.runner import to_device

    d_model = w.heads * w.head_dim
    n = w.query_frames
    x = to_device(G.hidden_frames(w, d_model, w.t0, n), "bf16")
    wq = to_device(G.qkv_weight(w, d_model), "bf16")
    fn = lambda: r.cache.qkv_rope_append(x, wq, r.q_rot, w.t0, n)  # noqa: E731
    us = back_to_back_us(fn, reps)
    flops = 2.0 * w.batch * w.query_rows * d_model * 3 * w.heads * w.head_dim
    tf = flops / (us * 1e-6) / 1e12
    # for scale, not part of the path: the library GEMM (torch.mm, hipBLASLt)
    # of the same shape with contiguous operands and a plain bf16 output
    # (no RoPE, no scatter into the ring)
    import torch

    x2 = x.reshape(-1, d_model)
    wt = wq.t().contiguous()
    out = torch.empty(x2.shape[0], wt.shape[1], device=x2.device, dtype=x2.dtype)
    lib_us = back_to_back_us(lambda: torch.mm(x2, wt, out=out), reps)
    del x2, wt, out
    return {"us": us, "d_model": d_model, "flops": flops, "tflops": tf, "frac_mfma": tf / PEAK_TFLOPS["bf16"],
            "library_gemm_us": lib_us, "library_gemm_frac_mfma": flops / (lib_us * 1e-6) / 1e12 / PEAK_TFLOPS["bf16"]}


def time_refresh_and_sink(r, w, reps=20):
    """HIP-event times of the RoPE refresh (every cached key's time pairs,
    one launch), of a one-frame sink update (its own launch), and of the
    chunk's append with and without its last frame also written into the
    sink (one launch), on the launch stream, after the timed steps (they
    change the cache state the steps ran on)."""
    eb = 2 if w.dtype == "bf16" else 4
    P, H, D, B = w.tokens_per_frame, w.heads, w.head_dim, w.batch
    cached_rows = w.n_slots * P  # every slot holds a frame in the steady state
    refresh_bytes = 2 * B * H * cached_rows * w.split[0] * eb
    sink_bytes = 4 * B * P * H * D * eb  # read k, v; write k_rot, v^T
    k1 = r.k[:, :P].contiguous()
    v1 = r.v[:, :P].contiguous()
    first = list(w.t0)
    nq = w.query_frames
    append_bytes = 6 * B * w.query_rows * H * D * eb
    fused_bytes = append_bytes + 2 * B * P * H * D * eb  # + the sink frame's k_rot and v^T writes
    res = {}
    cases = [
        # the sink update first: the refreshes move time positions below t0
        ("sink_update", lambda: r.cache.sink_update(k1, v1, first, 1), sink_bytes),
        # the chunk's append with its last frame also written into sink slot 0
        # (one launch): compare with "append" for the sink update's marginal cost
        ("append", lambda: r.cache.rope3d_append(r.q, r.q_rot, r.k, r.v, first, nq), append_bytes),
        ("append_with_sink", lambda: r.cache.rope3d_append_sink(r.q, r.q_rot, r.k, r.v, first, nq, nq - 1, 1),
         fused_bytes),
        ("rope_refresh", lambda: r.cache.rope_refresh([1] * B), refresh_bytes),
    ]
    if min(w.t0) < w.sink_frames:  # a chunk that lands in sink slots cannot also refresh them
        cases = [c for c in cases if c[0] != "append_with_sink"]
    for name, fn, nbytes in cases:
        us = back_to_back_us(fn, reps)
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"us": us, "algorithmic_bytes": nbytes, "gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS}
    if "append_with_sink" in res:
        res["append_with_sink"]["sink_marginal_us"] = res["append_with_sink"]["us"] - res["append"]["us"]
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the first ~20 launches after start-up run 3-10% slower than the steady
    # state a stream settles into (measured: 5 warm-up steps 0.646 ms, 30
    # steps 0.625 ms for the 480p attention on one box)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="wan1.3b-480p")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true", help="skip the amd-smi shader-clock sampling")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES bytes (counter calibration)")
    ap.add_argument("--ablations", action="store_true",
                    help="only print before/after timings of API-switchable design choices")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the multi-GPU sharding of this path "
              "is a design note, not a run.", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    # before anything touches the GPU
    clock_sampler = None if (args.ablations or args.no_clock) else start_clock_sampler()

    import torch

    from streaming_causal_video_amd import workloads as W
    from streaming_causal_video_amd.runner import StreamRunner

    w = W.WORKLOADS[args.workload]
    log(f"bench: {w.name}: {w.description}")
    if args.ablations:
        ablations(w)
        return
    r = StreamRunner(w, kv_splits=args.splits)
    r.fill()
    r.step()
    torch.cuda.synchronize()
    stamps = r.cache.views()["stamps"].cpu().numpy()
    pairs = visible_pairs(w, stamps)
    flops = 4 * w.head_dim * w.heads * pairs

    for _ in range(args.warmup):
        r.step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        r.append()
        ev[i][1].record()
        r.attend()
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = ev[0][0].elapsed_time(ev[K - 1][2])
    ms_per_step = total_ms / K
    append_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    attn_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    attn_each = sorted(e[1].elapsed_time(e[2]) for e in ev)
    pct = lambda q: attn_each[min(K - 1, int(q * (K - 1) + 0.5))]  # noqa: E731
    cold = cold_step_ms(r)
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    step_tflops = flops / (ms_per_step * 1e-3) / 1e12
    frames_per_s = w.batch * w.query_frames / (ms_per_step * 1e-3)
    eb = 2 if w.dtype == "bf16" else 4
    append_bytes = 6 * w.batch * w.query_rows * w.heads * w.head_dim * eb
    peak = PEAK_TFLOPS[w.dtype]
    m = MEASURED_TRAFFIC.get(w.name)
    traffic = None
    if m and m["source"] == kernel_source_hash() and m["kv_splits"] == r.splits:
        traffic = m["bytes_per_launch"]
    out = {
        "metric": "chunk-attn TFLOP/s (% MFMA bf16 peak) + latent frames/s, 1.3B-shape 480p",
        "value": step_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Philox N(0,1), rounded to the dtype)",
        "config": {
            "workload": w.name,
            "batch": w.batch,
            "heads": w.heads,
            "head_dim": w.head_dim,
            "query_rows": w.query_rows,
            "visible_keys_per_row": pairs // max(1, w.batch * w.query_rows),
            "t0": list(w.t0),
            "kv_splits": r.splits,
        },
        "pct_bf16_peak": 100.0 * step_tflops / peak,
        "latent_frames_per_s": frames_per_s,
        "attn_ms": attn_ms,
        "attn_ms_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "append_ms": append_ms,
        "cold": cold,
        "attn_kernel_tflops": attn_tflops,
        "append_gbs": append_bytes / (append_ms * 1e-3) / 1e9,
        "wall_s_timed": wall,
        "roofline": {
            "bound": "mfma",
            "achieved": attn_tflops,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": attn_tflops / peak,
            "traffic": traffic,
        },
    }
    if r.splits != 1:
        # key splits or the balanced schedule: the merge kernel is part of
        # the attention step (and of the events around it)
        out["attn_ms_includes_merge"] = True
    # the projection first: the refreshes move time positions below t0
    out["next_rows"] = {"qkv_rope_append": time_qkv(r, w)} if w.dtype == "bf16" else {}
    out["next_rows"].update(time_refresh_and_sink(r, w))
    out["sclk_under_load"] = None
    if clock_sampler:
        # after the timed steps: the same attention launch back to back for
        # 3 s, past the shader clock's start-up transient (reported beside
        # `attn_ms`, not used for `value`)
        window, sustained = load_window(r)
        out["sclk_under_load"] = read_clock_samples(clock_sampler, *window)
        out["attn_ms_sustained"] = dict(sustained, note="attention alone, launched back to back for 3 s after the timed steps (HIP events around all launches; includes the gaps between them)")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
