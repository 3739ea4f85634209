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


# ------------------------------------------- RoPE refresh and sink update ---
def _explicit_rot(x, pos):
    """Explicit block-diagonal rotation for split (2, 2, 2) (one pair per
    axis, omega_0 = 1, so each angle is the position itself)."""
    d = x.shape[-1]
    R = np.zeros((d, d))
    for blk, p in enumerate(pos):
        c, s = math.cos(float(p)), math.sin(float(p))
        R[2 * blk : 2 * blk + 2, 2 * blk : 2 * blk + 2] = [[c, -s], [s, c]]
    return R @ x


def check_refresh_keeps_attention():
    """A RoPE refresh changes no output: two caches fed the same streams, one
    of them refreshed twice along the way, give the same O and lse on every
    chunk (scores depend only on differences of time positions, and the
    refresh moves keys and later queries by the same amount)."""
    rng = np.random.default_rng(61)
    spec = O.CacheSpec(batch=2, heads=2, head_dim=12, split=(4, 4, 4), base=10000.0, grid_h=2, grid_w=3,
                       sink_frames=1, window_frames=4, chunk_frames=2)
    P, H, d, C = 6, 2, 12, 2
    plain, fresh = O.OracleCache(spec), O.OracleCache(spec)
    sk, sv = rng.standard_normal((2, P, H, d)), rng.standard_normal((2, P, H, d))
    plain.init(sk, sv)
    fresh.init(sk, sv)
    refresh_at = {3: [5, 1000], 6: [1, 5]}
    for step in range(9):
        t0 = [1 + C * step, 1000 + C * step]
        q, k, v = (rng.standard_normal((2, C * P, H, d)) for _ in range(3))
        if step in refresh_at:
            fresh.rope_refresh(refresh_at[step])
        qa = plain.rope3d_append(q, k, v, t0, C)
        qb = fresh.rope3d_append(q, k, v, t0, C)
        oa, la = plain.chunk_attention(qa, t0, C)
        ob, lb = fresh.chunk_attention(qb, t0, C)
        assert np.max(np.abs(oa - ob)) <= 1e-9, step
        assert np.max(np.abs(la - lb)) <= 1e-9, step
        assert np.array_equal(plain.stamps, fresh.stamps)
    assert list(fresh.pos_offset) == [6, 1005]


def check_refresh_equals_rotation_at_earlier_time():
    """After refresh(delta) every cached key equals its raw key rotated by
    explicit rotation matrices at time position (frame - delta), sink
    included, and the next append rotates at (frame - delta) as well."""
    rng = np.random.default_rng(62)
    spec = O.CacheSpec(batch=1, heads=1, head_dim=6, split=(2, 2, 2), base=10000.0, grid_h=2, grid_w=2,
                       sink_frames=1, window_frames=2, chunk_frames=1)
    cache = O.OracleCache(spec)
    raw = {}
    for g in range(5):
        q, k, v = (rng.standard_normal((1, 4, 1, 6)) for _ in range(3))
        raw[g] = k
        cache.rope3d_append(q, k, v, [g], 1)
    cache.rope_refresh([3])
    for slot in range(spec.n_slots):
        g = int(cache.stamps[0, slot])
        for p in range(4):
            want = _explicit_rot(raw[g][0, p, 0], (g - 3, p // 2, p % 2))
            assert np.max(np.abs(cache.k[0][slot][p, 0] - want)) <= 1e-12, (slot, g, p)
    x = rng.standard_normal((1, 4, 1, 6))
    y = cache.rope3d_apply(x, [5], 1)
    for p in range(4):
        assert np.max(np.abs(y[0, p, 0] - _explicit_rot(x[0, p, 0], (2, p // 2, p % 2)))) <= 1e-12


def _sink_brute(n_calls, chunks_per_call, update_call, update_frame_in_call, seed):
    """Stream of single-frame chunks (C = 1, S_f = 1, W = 2, d = 6), each call
    appending ``chunks_per_call`` frames; in call ``update_call`` the sink
    takes the k/v of that call's frame ``update_frame_in_call``.  Every
    chunk's output equals brute-force attention over an explicit key list --
    the sink entry (seen by a chunk iff the chunk does not end before its
    frame, whatever the window) plus the window frames -- with keys rotated
    by explicit matrices at their own frames; the update leaves the ring
    untouched."""
    rng = np.random.default_rng(seed)
    d, P, W, Sf, n = 6, 4, 2, 1, chunks_per_call
    spec = O.CacheSpec(batch=1, heads=1, head_dim=d, split=(2, 2, 2), base=10000.0, grid_h=2, grid_w=2,
                       sink_frames=Sf, window_frames=W, chunk_frames=1, max_query_chunks=n)
    cache = O.OracleCache(spec)
    hist = {}  # frame -> (rotated keys, values)
    sink = None  # (frame, keys, values)
    for call in range(n_calls):
        t0 = call * n
        q, k, v = (rng.standard_normal((1, n * P, 1, d)) for _ in range(3))
        q_rot = cache.rope3d_append(q, k, v, [t0], n)
        for f in range(n):
            g = t0 + f
            hist[g] = ([_explicit_rot(k[0, f * P + p, 0], (g, p // 2, p % 2)) for p in range(P)],
                       [v[0, f * P + p, 0] for p in range(P)])
        if call == 0:
            sink = (0, *hist[0])
        if call == update_call:
            ring_k = {s_: cache.k[0][s_].copy() for s_ in range(Sf, spec.n_slots) if s_ in cache.k[0]}
            ring_stamps = cache.stamps[0, Sf:].copy()
            u = update_frame_in_call
            cache.sink_update(k[:, u * P : (u + 1) * P], v[:, u * P : (u + 1) * P], [t0 + u], 1)
            sink = (t0 + u, *hist[t0 + u])
            assert np.array_equal(cache.stamps[0, Sf:], ring_stamps)
            for s_, kk in ring_k.items():
                assert np.array_equal(cache.k[0][s_], kk)
            assert cache.stamps[0, 0] == t0 + u
        o, _ = cache.chunk_attention(q_rot, [t0], n)
        for f in range(n):
            g = t0 + f
            entries = []
            if sink[0] <= g:
                entries += list(zip(sink[1], sink[2]))
            for fr in range(max(Sf, g - W), g + 1):
                entries += list(zip(*hist[fr]))
            for p in range(P):
                qr = _explicit_rot(q[0, f * P + p, 0], (g, p // 2, p % 2))
                scores = [sum(qr[c] * kk[c] for c in range(d)) / math.sqrt(d) for kk, _ in entries]
                m = max(scores)
                e = [math.exp(x - m) for x in scores]
                tot = sum(e)
                ob = sum((e[j] / tot) * entries[j][1] for j in range(len(e)))
                assert np.max(np.abs(o[0, f * P + p, 0] - ob)) <= 1e-12, (call, f, p)


def check_sink_update_brute_force():
    # one chunk per call; the sink takes the newest frame at frame 5
    _sink_brute(12, 1, 5, 0, 63)
    # two chunks per call; the sink takes the second chunk's frame, which the
    # first chunk of the same call must not see
    _sink_brute(7, 2, 3, 1, 65)


def check_sink_update_with_the_sink_itself_is_a_no_op():
    """Replacing the sink by the initial frame's own k/v changes nothing."""
    rng = np.random.default_rng(64)
    spec = O.CacheSpec(batch=1, heads=2, head_dim=12, split=(4, 4, 4), base=10000.0, grid_h=2, grid_w=2,
                       sink_frames=1, window_frames=3, chunk_frames=2)
    a, b = O.OracleCache(spec), O.OracleCache(spec)
    sk, sv = rng.standard_normal((1, 4, 2, 12)), rng.standard_normal((1, 4, 2, 12))
    a.init(sk, sv)
    b.init(sk, sv)
    b.sink_update(sk, sv, [0], 1)
    for step in range(4):
        t0 = [1 + 2 * step]
        q, k, v = (rng.standard_normal((1, 8, 2, 12)) for _ in range(3))
        oa, la = a.chunk_attention(a.rope3d_append(q, k, v, t0, 2), t0, 2)
        ob, lb = b.chunk_attention(b.rope3d_append(q, k, v, t0, 2), t0, 2)
        assert np.max(np.abs(oa - ob)) <= 1e-15 and np.max(np.abs(la - lb)) <= 1e-15
        assert np.array_equal(a.stamps, b.stamps)


# ------------------------------------------------------- QKV projection ---
def check_qkv_projection_brute_force():
    """Triple loops over (token, output feature, input feature), with the
    feature order written out: q head h dim i is weight row h*d + i, k the
    same after H*d rows, v after 2*H*d rows."""
    rng = np.random.default_rng(71)
    B, N, Dm, H, d = 2, 3, 5, 2, 4
    x = rng.standard_normal((B, N, Dm))
    w = rng.standard_normal((3 * H * d, Dm))
    q, k, v = O.qkv_project(x, w, H, d)
    for b in range(B):
        for n in range(N):
            for h in range(H):
                for i in range(d):
                    for which, out in enumerate((q, k, v)):
                        row = which * H * d + h * d + i
                        want = sum(x[b, n, c] * w[row, c] for c in range(Dm))
                        assert abs(out[b, n, h, i] - want) <= 1e-12, (which, b, n, h, i)


def check_qkv_projection_selects_columns():
    """A weight of one-hot rows copies the chosen input features exactly."""
    rng = np.random.default_rng(72)
    B, N, Dm, H, d = 1, 4, 7, 1, 2
    x = rng.standard_normal((B, N, Dm))
    pick = [3, 0, 6, 6, 1, 2]  # input feature of each of the 3*H*d rows
    w = np.zeros((3 * H * d, Dm))
    for r, c in enumerate(pick):
        w[r, c] = 1.0
    q, k, v = O.qkv_project(x, w, H, d)
    assert np.array_equal(q[0, :, 0], x[0][:, [3, 0]])
    assert np.array_equal(k[0, :, 0], x[0][:, [6, 6]])
    assert np.array_equal(v[0, :, 0], x[0][:, [1, 2]])


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
    check_refresh_keeps_attention,
    check_refresh_equals_rotation_at_earlier_time,
    check_sink_update_brute_force,
    check_sink_update_with_the_sink_itself_is_a_no_op,
    check_qkv_projection_brute_force,
    check_qkv_projection_selects_columns,
]
