"""Checks that pin the fp64 oracle to facts outside itself.

Each ``check_*`` raises AssertionError when the oracle disagrees with:
hand-derived golden values (tests/golden, each file states its source),
closed forms, high-precision mpmath evaluation, brute force with explicit
loops and rotation matrices, a library routine (torch SDPA in float64), or
an invariant of the mathematics.  The functions look the oracle up through
the module object at call time, so a test can plant a mistake in the oracle
(monkeypatch) and confirm that some check catches it.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import mpmath
import numpy as np

from oracle import scv_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- RoPE -----
def check_golden_unit_vectors():
    """Unit vectors rotated by hand (pairing, sign, axis order, ladder)."""
    for r in _rows("rope_unit_vectors.txt"):
        dim, pt, ph, pw, a, va, b, vb = int(r[0]), int(r[1]), int(r[2]), int(r[3]), int(r[4]), float(r[5]), int(r[6]), float(r[7])
        x = np.zeros((1, 1, 24))
        x[0, 0, dim] = 1.0
        y = O.rope3d(x, np.array([pt]), np.array([ph]), np.array([pw]), (8, 8, 8), 10000.0)[0, 0]
        exp = np.zeros(24)
        exp[a], exp[b] = va, vb
        assert np.max(np.abs(y - exp)) <= 2e-15, (r, y)


def check_frequency_ladder():
    """omega_j = base^(-2j/d): omega_0 = 1, constant ratio base^(-2/d),
    omega_{d/4} = base^(-1/2), and every entry within 1 ulp of a 50-digit
    mpmath evaluation of the same power."""
    mpmath.mp.dps = 50
    for base, d in ((10000.0, 44), (10000.0, 42), (10000.0, 24), (10000.0, 20), (10000.0, 8), (500.0, 16), (10000.0, 2)):
        w = O.rope_frequencies(d, base)
        assert w.shape == (d // 2,) and w.dtype == np.float64
        assert w[0] == 1.0
        for j in range(d // 2):
            ulp = mpmath.mpf(float(np.spacing(w[j])))
            # the value of the fp64 exponent -(2j)/d, within 1 ulp ...
            e64 = -(2.0 * j) / float(d)
            ref = mpmath.power(mpmath.mpf(base), mpmath.mpf(e64))
            assert abs(mpmath.mpf(float(w[j])) - ref) <= ulp, (base, d, j)
            # ... and of the exact ladder base^(-2j/d) within the few ulps
            # that rounding the exponent costs (ln(base) * 2^-53 relative)
            exact = mpmath.power(mpmath.mpf(base), mpmath.mpf(-2 * j) / d)
            assert abs(mpmath.mpf(float(w[j])) - exact) <= 16 * ulp, (base, d, j)
        if d % 4 == 0 and d >= 4:
            assert abs(w[d // 4] - base ** -0.5) <= 1e-16 * base ** -0.5 * 4


def check_angles_are_exact_fp64_products():
    """theta = fl64(pos * omega) exactly: compare with the correctly rounded
    product of the exact rationals (Fraction -> float rounds correctly)."""
    poss = np.array([0, 1, 2, 3, 37, 999, 1000, 1002, 5000, 20002, 100000, 100002, 2**31 - 1, 2**40 - 1], dtype=np.int64)
    for d in (44, 42, 24, 20):
        th = O.rope_angles(poss, d, 10000.0)
        om = O.rope_frequencies(d, 10000.0)
        for i, p in enumerate(poss):
            for j in range(d // 2):
                exact = float(Fraction(int(p)) * Fraction(float(om[j])))
                assert th[i, j] == exact, (p, j)


def _mp_round_f32(v):
    """Nearest float32 to an mpmath value, and whether v is within 2^-40
    (relative) of a float32 rounding midpoint."""
    c = np.float32(float(v))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(cands, key=lambda f: abs(mpmath.mpf(float(f)) - v))
    near_mid = False
    for f in cands:
        mid = (mpmath.mpf(float(best)) + mpmath.mpf(float(f))) / 2
        if f != best and abs(v - mid) <= abs(v) * mpmath.mpf(2) ** -40:
            near_mid = True
    return best, near_mid


def check_tables_match_high_precision():
    """fp32 cos/sin tables equal the float32 rounding of the 40-digit cos/sin
    of the exact fp64 angle (entries within 2^-40 of a float32 midpoint are
    counted and skipped; none are expected)."""
    mpmath.mp.dps = 40
    t0 = [0, 37, 1000, 100000, 2**40 - 3]
    tabs = O.rope_cos_sin_tables(t0, 3, 5, 7, (44, 42, 42), 10000.0)
    assert tabs["t"].shape == (5, 3, 22, 2) and tabs["t"].dtype == np.float32
    assert tabs["h"].shape == (5, 21, 2) and tabs["w"].shape == (7, 21, 2)
    near = 0
    for name, pos, d in (
        ("t", np.array(t0)[:, None] + np.arange(3)[None, :], 44),
        ("h", np.arange(5), 42),
        ("w", np.arange(7), 42),
    ):
        om = O.rope_frequencies(d, 10000.0)
        for idx in np.ndindex(*np.shape(pos)):
            p = int(np.asarray(pos)[idx])
            for j in range(d // 2):
                th = mpmath.mpf(float(Fraction(p) * Fraction(float(om[j]))))
                for k, fn in ((0, mpmath.cos), (1, mpmath.sin)):
                    ref, nm = _mp_round_f32(fn(th))
                    if nm:
                        near += 1
                        continue
                    got = tabs[name][idx + (j, k)]
                    assert got == ref, (name, idx, j, k, got, ref)
    assert near == 0


def check_rope_norm_identity_complex():
    """Pair norms preserved; position 0 is the identity; agrees with the
    complex form (x + iy) e^{i theta} evaluated with math.cos/math.sin."""
    rng = np.random.default_rng(11)
    split = (44, 42, 42)
    x = rng.standard_normal((9, 3, 128))
    t = np.array([0, 1, 5, 1000, 100000, 7, 2**33, 3, 0])
    h = np.array([0, 2, 29, 4, 0, 11, 3, 44, 0])
    w = np.array([0, 51, 3, 0, 79, 5, 1, 2, 0])
    y = O.rope3d(x, t, h, w, split, 10000.0)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.max(np.abs(nx - ny)) <= 1e-12
    assert np.array_equal(y[0], x[0]) and np.array_equal(y[-1], x[-1])
    lo = 0
    for width, pos in zip(split, (t, h, w)):
        for n in range(x.shape[0]):
            for j in range(width // 2):
                om = math.pow(10000.0, -(2.0 * j) / width)
                th = float(pos[n]) * om
                z = (x[n, :, lo + 2 * j] + 1j * x[n, :, lo + 2 * j + 1]) * complex(math.cos(th), math.sin(th))
                assert np.max(np.abs(z.real - y[n, :, lo + 2 * j])) <= 1e-13
                assert np.max(np.abs(z.imag - y[n, :, lo + 2 * j + 1])) <= 1e-13
        lo += width


def check_rope_relative_position():
    """<R(p1) q, R(p2) k> depends only on p1 - p2, per axis: shifting every
    position by the same offset leaves the score unchanged."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((6, 2, 64))
    k = rng.standard_normal((6, 2, 64))
    split = (24, 20, 20)
    tq, hq, wq = np.array([3, 9, 40, 0, 12, 37]), np.array([0, 1, 2, 3, 0, 1]), np.array([3, 2, 1, 0, 3, 2])
    tk, hk, wk = np.array([0, 9, 33, 1, 2, 38]), np.array([3, 3, 0, 1, 2, 0]), np.array([0, 1, 2, 3, 1, 1])
    base = np.einsum("nhd,nhd->nh", O.rope3d(q, tq, hq, wq, split, 1e4), O.rope3d(k, tk, hk, wk, split, 1e4))
    for dt, dh, dw in ((1, 0, 0), (37, 0, 0), (1000, 0, 0), (100000, 0, 0), (0, 5, 0), (0, 0, 7), (250, 3, 11)):
        s = np.einsum(
            "nhd,nhd->nh",
            O.rope3d(q, tq + dt, hq + dh, wq + dw, split, 1e4),
            O.rope3d(k, tk + dt, hk + dh, wk + dw, split, 1e4),
        )
        assert np.max(np.abs(s - base)) <= 1e-9, (dt, dh, dw)


def check_rope_rotation_matrix_brute_force():
    """Against an explicit d x d block-diagonal rotation matrix per token."""
    rng = np.random.default_rng(3)
    split = (2, 2, 2)
    x = rng.standard_normal((4, 2, 6))
    t, h, w = np.array([0, 1, 7, 12]), np.array([1, 0, 1, 1]), np.array([0, 1, 1, 0])
    y = O.rope3d(x, t, h, w, split, 10000.0)
    for n in range(4):
        R = np.zeros((6, 6))
        for blk, pos in enumerate((t[n], h[n], w[n])):
            th = float(pos) * 1.0  # one pair per axis: omega_0 = 1
            c, s = math.cos(th), math.sin(th)
            R[2 * blk : 2 * blk + 2, 2 * blk : 2 * blk + 2] = [[c, -s], [s, c]]
        for hh in range(2):
            assert np.max(np.abs(R @ x[n, hh] - y[n, hh])) <= 1e-14


# ----------------------------------------------------------- ring / mask ---
def check_golden_ring_slots():
    for r in _rows("ring_slots.txt"):
        sf, R, g, slot = map(int, r)
        assert O.frame_slot(g, sf, R) == slot, r


def check_golden_visible_counts():
    for r in _rows("visible_keys.txt"):
        sf, W, C, s, n = map(int, r)
        got = sum(O.frame_visible(g, s, C, sf, W) for g in range(0, s + C + 5))
        assert got == n, (r, got)


def check_token_positions():
    """Frame-major, row-major token order on a 3 x 5 grid."""
    t, h, w = O.token_positions(40, 2, 3, 5)
    assert list(t[:15]) == [40] * 15 and list(t[15:]) == [41] * 15
    assert list(h[:15]) == [0] * 5 + [1] * 5 + [2] * 5
    assert list(w[:7]) == [0, 1, 2, 3, 4, 0, 1]


# ------------------------------------------------------------ attention ----
def _brute_attention(q, k, v, scale):
    """Double loops: scores, explicit max / exp / sum, weighted sum."""
    M, d = q.shape
    N = k.shape[0]
    o = np.zeros((M, v.shape[1]))
    lse = np.zeros(M)
    for i in range(M):
        s = [sum(q[i, c] * k[j, c] for c in range(d)) * scale for j in range(N)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        tot = sum(e)
        for j in range(N):
            o[i] += (e[j] / tot) * v[j]
        lse[i] = m + math.log(tot)
    return o, lse


def check_attention_brute_force():
    rng = np.random.default_rng(17)
    for M, N, d in ((3, 5, 4), (7, 1, 6), (4, 13, 8)):
        q, k, v = rng.standard_normal((M, d)), rng.standard_normal((N, d)), rng.standard_normal((N, d))
        o, lse = O.attention(q, k, v, 1.0 / math.sqrt(d))
        ob, lb = _brute_attention(q, k, v, 1.0 / math.sqrt(d))
        assert np.max(np.abs(o - ob)) <= 1e-12 and np.max(np.abs(lse - lb)) <= 1e-12


def check_attention_sdpa():
    """torch scaled_dot_product_attention in float64 on the CPU."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(23)
    M, N, d = 20, 37, 16
    q, k, v = rng.standard_normal((M, d)), rng.standard_normal((N, d)), rng.standard_normal((N, d))
    o, _ = O.attention(q, k, v, 1.0 / math.sqrt(d))
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], scale=1.0 / math.sqrt(d)
    )[0].numpy()
    assert np.max(np.abs(o - ref)) <= 1e-12


def check_attention_closed_forms():
    rng = np.random.default_rng(29)
    M, N, d = 6, 11, 8
    q, k = rng.standard_normal((M, d)), rng.standard_normal((N, d))
    # V = identity: O is the probability matrix itself; rows sum to 1.
    o, _ = O.attention(q, k, np.eye(N), 0.3)
    assert np.all(o >= 0) and np.max(np.abs(o.sum(axis=1) - 1.0)) <= 1e-12
    # constant v rows -> O is that row
    c = rng.standard_normal(d)
    o, _ = O.attention(q, k, np.tile(c, (N, 1)), 0.3)
    assert np.max(np.abs(o - c)) <= 1e-12
    # q = 0 -> uniform weights: mean of v, lse = log N
    v = rng.standard_normal((N, d))
    o, lse = O.attention(np.zeros((M, d)), k, v, 0.3)
    assert np.max(np.abs(o - v.mean(axis=0))) <= 1e-12
    assert np.max(np.abs(lse - math.log(N))) <= 1e-12
    # one key far above the rest -> O ~ its v
    kk = rng.standard_normal((N, d)) * 0.01
    qq = np.ones((1, d))
    kk[4] = 50.0 * np.ones(d) / d
    o, _ = O.attention(qq, kk, v, 1.0)
    assert np.max(np.abs(o[0] - v[4])) <= 1e-14
    # no keys -> O = 0, lse = -inf
    o, lse = O.attention(q, np.zeros((0, d)), np.zeros((0, d)), 0.3)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def check_merge_identity():
    rng = np.random.default_rng(31)
    M, N, d = 9, 40, 8
    q, k, v = rng.standard_normal((M, d)), rng.standard_normal((N, d)), rng.standard_normal((N, d))
    full, lse = O.attention(q, k, v, 0.35)
    cuts = [0, 7, 7, 25, 40]  # includes an empty part
    parts = [O.attention(q, k[a:b], v[a:b], 0.35) for a, b in zip(cuts[:-1], cuts[1:])]
    om, lm = O.merge_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    assert np.max(np.abs(om - full)) <= 1e-13 and np.max(np.abs(lm - lse)) <= 1e-13


# --------------------------------------------------- the streaming cache ---
def _stream_check(spec, n_chunks, seed):
    """Stream from t0 = 0; every call's output from the ring equals masked
    full-history attention (the definition the rolling cache implements)."""
    rng = np.random.default_rng(seed)
    P, C, H, d = spec.tokens_per_frame, spec.chunk_frames, spec.heads, spec.head_dim
    k_hist, v_hist = {}, {}
    cache = O.OracleCache(spec)
    nq = spec.max_query_chunks * C
    for step in range(n_chunks):
        t0 = step * nq
        q = rng.standard_normal((1, nq * P, H, d))
        k = rng.standard_normal((1, nq * P, H, d))
        v = rng.standard_normal((1, nq * P, H, d))
        q_rot = cache.rope3d_append(q, k, v, [t0], nq)
        o, lse = cache.chunk_attention(q_rot, [t0], nq)
        k_rot = cache.rope3d_apply(k, [t0], nq)
        for f in range(nq):
            k_hist[t0 + f] = k_rot[0, f * P : (f + 1) * P]
            v_hist[t0 + f] = v[0, f * P : (f + 1) * P]
        for c in range(spec.max_query_chunks):
            rows = slice(c * C * P, (c + 1) * C * P)
            of, lf = O.full_history_attention(spec, q_rot[0, rows], k_hist, v_hist, t0 + c * C)
            assert np.max(np.abs(o[0, rows] - of)) <= 1e-12, (step, c)
            assert np.max(np.abs(lse[0, :, rows] - lf)) <= 1e-12, (step, c)
        # stamps: each slot holds the latest frame that maps to it
        for slot in range(spec.n_slots):
            frames = [g for g in k_hist if O.frame_slot(g, spec.sink_frames, spec.ring_frames) == slot]
            assert cache.stamps[0, slot] == (max(frames) if frames else -1)


def check_rolling_cache_equals_masked_full_attention():
    base = dict(batch=1, heads=2, head_dim=6, split=(2, 2, 2), base=10000.0, grid_h=2, grid_w=2)
    _stream_check(O.CacheSpec(sink_frames=1, window_frames=4, chunk_frames=2, **base), 20, 1)
    _stream_check(O.CacheSpec(sink_frames=1, window_frames=5, chunk_frames=2, **base), 20, 2)
    _stream_check(O.CacheSpec(sink_frames=2, window_frames=3, chunk_frames=1, **base), 15, 3)
    _stream_check(O.CacheSpec(sink_frames=1, window_frames=4, chunk_frames=2, max_query_chunks=2, **base), 12, 4)


def _brute_stream(n_chunks):
    """Brute force of a whole stream (d = 6, split 2/2/2, grid 2x2, C = 1,
    S_f = 1, W = 2): explicit rotation matrices, score double loops, explicit
    exp/sum loops, and a 0/1 mask over the full history."""
    rng = np.random.default_rng(99)
    d, P, H, W, Sf = 6, 4, 1, 2, 1
    spec = O.CacheSpec(batch=1, heads=H, head_dim=d, split=(2, 2, 2), base=10000.0, grid_h=2, grid_w=2,
                       sink_frames=Sf, window_frames=W, chunk_frames=1)
    cache = O.OracleCache(spec)
    hist_k, hist_v = [], []
    for g in range(n_chunks):
        q = rng.standard_normal((1, P, H, d))
        k = rng.standard_normal((1, P, H, d))
        v = rng.standard_normal((1, P, H, d))
        q_rot = cache.rope3d_append(q, k, v, [g], 1)
        o, _ = cache.chunk_attention(q_rot, [g], 1)

        def rot(x, pos):
            R = np.zeros((d, d))
            for blk, p in enumerate(pos):
                c, s = math.cos(float(p)), math.sin(float(p))
                R[2 * blk : 2 * blk + 2, 2 * blk : 2 * blk + 2] = [[c, -s], [s, c]]
            return R @ x

        for p in range(P):
            hist_k.append((g, rot(k[0, p, 0], (g, p // 2, p % 2))))
            hist_v.append(v[0, p, 0])
        for p in range(P):
            qr = rot(q[0, p, 0], (g, p // 2, p % 2))
            scores, keep = [], []
            for (gk, kr) in hist_k:
                vis = 1 if (gk < g + 1 and (gk < Sf or gk >= g - W)) else 0
                keep.append(vis)
                scores.append(sum(qr[c] * kr[c] for c in range(d)) / math.sqrt(d))
            m = max(s for s, kp in zip(scores, keep) if kp)
            e = [math.exp(s - m) if kp else 0.0 for s, kp in zip(scores, keep)]
            tot = sum(e)
            ob = sum((e[j] / tot) * hist_v[j] for j in range(len(e)))
            assert np.max(np.abs(o[0, p, 0] - ob)) <= 1e-12, (g, p)


def check_stream_brute_force():
    _brute_stream(12)


def check_shift_invariance_of_attention():
    """Shifting every time index (sink included) by the same offset leaves
    the chunk's output unchanged."""
    rng = np.random.default_rng(41)
    split, P = (24, 20, 20), 16
    frames = [0, 33, 34, 35, 36, 37, 38]
    q = rng.standard_normal((2 * P, 2, 64))
    ks = {g: rng.standard_normal((P, 2, 64)) for g in frames}
    vs = {g: rng.standard_normal((P, 2, 64)) for g in frames}

    def run(delta):
        tq, hq, wq = O.token_positions(37 + delta, 2, 4, 4)
        qr = O.rope3d(q, tq, hq, wq, split, 1e4)
        K = np.concatenate([O.rope3d(ks[g], *O.token_positions(g + delta, 1, 4, 4), split, 1e4) for g in frames])
        V = np.concatenate([vs[g] for g in frames])
        return np.stack([O.attention(qr[:, h], K[:, h], V[:, h], 0.125)[0] for h in range(2)])

    ref = run(0)
    for delta in (1, 37, 1000, 100000):
        assert np.max(np.abs(run(delta) - ref)) <= 1e-9, delta


ALL_CHECKS = [
    check_golden_unit_vectors,
    check_frequency_ladder,
    check_angles_are_exact_fp64_products,
    check_tables_match_high_precision,
    check_rope_norm_identity_complex,
    check_rope_relative_position,
    check_rope_rotation_matrix_brute_force,
    check_golden_ring_slots,
    check_golden_visible_counts,
    check_token_positions,
    check_attention_brute_force,
    check_attention_sdpa,
    check_attention_closed_forms,
    check_merge_identity,
    check_rolling_cache_equals_masked_full_attention,
    check_stream_brute_force,
    check_shift_invariance_of_attention,
]
