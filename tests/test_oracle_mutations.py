"""Plant plausible mistakes in the oracle (CPU only) and confirm the pins
catch each one: the pins are only worth something if they fail on a wrong
sign, a dropped term, a swapped index or a transposed operand."""
import math

import numpy as np
import pytest

import oracle_pins as pins
from oracle import scv_oracle as O

_orig_rope3d = O.rope3d
_orig_attention = O.attention
_orig_frame_visible = O.frame_visible
_orig_frame_slot = O.frame_slot
_orig_qkv = O.qkv_project


def _rope3d_variant(sign=1.0, half_split=False, order=(0, 1, 2)):
    def rope3d(x, pos_t, pos_h, pos_w, split, base):
        x = np.asarray(x, dtype=np.float64)
        out = np.empty_like(x)
        pos = (pos_t, pos_h, pos_w)
        lo = 0
        for a in order:
            width = split[a]
            th = O.rope_angles(pos[a], width, base)
            c, s = np.cos(th)[:, None, :], sign * np.sin(th)[:, None, :]
            if half_split:
                xe, xo = x[:, :, lo : lo + width // 2], x[:, :, lo + width // 2 : lo + width]
                out[:, :, lo : lo + width // 2] = xe * c - xo * s
                out[:, :, lo + width // 2 : lo + width] = xe * s + xo * c
            else:
                xe, xo = x[:, :, lo : lo + width : 2], x[:, :, lo + 1 : lo + width : 2]
                out[:, :, lo : lo + width : 2] = xe * c - xo * s
                out[:, :, lo + 1 : lo + width : 2] = xe * s + xo * c
            lo += width
        return out

    return rope3d


def _attention_variant(kind):
    def attention(q, k, v, scale):
        if kind == "no_scale":
            return _orig_attention(q, k, v, 1.0)
        if kind == "transposed_v":
            o, lse = _orig_attention(q, k, v, scale)
            if k.shape[0] == 0:
                return o, lse
            s = (np.asarray(q) @ np.asarray(k).T) * scale
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            vv = np.asarray(v)
            if vv.shape[0] == vv.shape[1]:
                return p @ vv.T, lse
            return p @ vv[::-1], lse
        if kind == "lse_no_max":
            o, lse = _orig_attention(q, k, v, scale)
            if k.shape[0] == 0:
                return o, lse
            s = (np.asarray(q) @ np.asarray(k).T) * scale
            return o, lse - s.max(axis=1)
        if kind == "drop_last_key":
            if k.shape[0] > 1:
                return _orig_attention(q, k[:-1], v[:-1], scale)
            return _orig_attention(q, k, v, scale)
        raise ValueError(kind)

    return attention


def _frequencies_variant(kind):
    def rope_frequencies(d_axis, base):
        j = np.arange(d_axis // 2, dtype=np.float64)
        if kind == "exp_j_over_d":
            return np.power(float(base), -j / d_axis)
        if kind == "exp_plus_one":
            return np.power(float(base), -(2.0 * j + 1.0) / d_axis)
        raise ValueError(kind)

    return rope_frequencies


def _refresh_variant(kind):
    def rope_refresh(self, delta):
        s = self.spec
        for b in range(s.batch):
            dlt = int(delta[b])
            for slot, kk in self.k[b].items():
                if kind == "skips_sink" and slot < s.sink_frames:
                    continue
                n = kk.shape[0]
                t = np.full(n, dlt if kind == "wrong_sign" else -dlt, dtype=np.int64)
                hw = t if kind == "turns_all_axes" else np.zeros(n, dtype=np.int64)
                self.k[b][slot] = O.rope3d(kk, t, hw, hw, s.split, s.base)
            if kind != "forgets_offset":
                self.pos_offset[b] += dlt

    return rope_refresh


def _sink_update_at_slot_time(self, k, v, first_frame, n_frames):
    # rotates the new sink at the time of the slot it replaces, not its frame
    s = self.spec
    P = s.tokens_per_frame
    k_rot = self.rope3d_apply(k, [0] * s.batch, n_frames)
    for b in range(s.batch):
        for j in range(n_frames):
            self.k[b][j] = k_rot[b, j * P : (j + 1) * P]
            self.v[b][j] = np.asarray(v[b, j * P : (j + 1) * P], dtype=np.float64)
            self.stamps[b, j] = int(first_frame[b]) + j


def _qkv_transposed(x, w):
    # reads the weight as [d_model, 3*H*d] in memory order (a transposed operand)
    wt = np.asarray(w).reshape(-1)[: w.size].reshape(w.shape[1], w.shape[0])
    return np.asarray(x) @ wt


def _split(y, x, H, d):
    y = y.reshape(x.shape[0], x.shape[1], 3, H, d)
    return y[:, :, 0], y[:, :, 1], y[:, :, 2]


def _qkv_swapped(x, w, H, d):
    q, k, v = _orig_qkv(x, w, H, d)
    return q, v, k


def _qkv_interleaved(x, w, H, d):
    # features taken as (head, q/k/v, dim) instead of (q/k/v, head, dim)
    y = np.asarray(x) @ np.asarray(w).T
    y = y.reshape(x.shape[0], x.shape[1], H, 3, d)
    return y[:, :, :, 0], y[:, :, :, 1], y[:, :, :, 2]


MUTATIONS = {
    "rope_sin_sign": ("rope3d", _rope3d_variant(sign=-1.0)),
    "rope_half_split_pairs": ("rope3d", _rope3d_variant(half_split=True)),
    "rope_axis_order_hwt": ("rope3d", _rope3d_variant(order=(1, 2, 0))),
    "freq_exponent_j_over_d": ("rope_frequencies", _frequencies_variant("exp_j_over_d")),
    "freq_exponent_off_by_one": ("rope_frequencies", _frequencies_variant("exp_plus_one")),
    "angles_in_fp32": (
        "rope_angles",
        lambda pos, d, base: (np.asarray(pos, np.float32)[..., None] * O.rope_frequencies(d, base).astype(np.float32)).astype(np.float64),
    ),
    "slot_without_sink_offset": ("frame_slot", lambda g, sf, R: g if g < sf else g % R),
    "slot_sink_not_pinned": ("frame_slot", lambda g, sf, R: sf + (g % R)),
    "window_off_by_one": ("frame_visible", lambda g, s, C, sf, W: g >= 0 and g < s + C and (g < sf or g > s - W)),
    "not_block_causal": ("frame_visible", lambda g, s, C, sf, W: g >= 0 and (g < sf or g >= s - W)),
    "causal_drops_own_chunk": ("frame_visible", lambda g, s, C, sf, W: g >= 0 and g < s and (g < sf or g >= s - W)),
    "no_sink": ("frame_visible", lambda g, s, C, sf, W: g >= 0 and g < s + C and g >= s - W),
    "attention_no_scale": ("attention", _attention_variant("no_scale")),
    "attention_transposed_v": ("attention", _attention_variant("transposed_v")),
    "attention_lse_dropped_max": ("attention", _attention_variant("lse_no_max")),
    "attention_drops_a_key": ("attention", _attention_variant("drop_last_key")),
    "refresh_wrong_sign": ("OracleCache.rope_refresh", _refresh_variant("wrong_sign")),
    "refresh_forgets_offset": ("OracleCache.rope_refresh", _refresh_variant("forgets_offset")),
    "refresh_skips_sink": ("OracleCache.rope_refresh", _refresh_variant("skips_sink")),
    "refresh_turns_all_axes": ("OracleCache.rope_refresh", _refresh_variant("turns_all_axes")),
    "sink_update_at_slot_time": ("OracleCache.sink_update", _sink_update_at_slot_time),
    "sink_follows_window": ("slot_visible", lambda slot, g, s, C, sf, W: O.frame_visible(g, s, C, sf, W)),
    "sink_not_causal": ("slot_visible", lambda slot, g, s, C, sf, W: g >= 0 if slot < sf else
                        O.frame_visible(g, s, C, sf, W)),
    "qkv_weight_not_transposed": ("qkv_project", lambda x, w, H, d: _split(_qkv_transposed(x, w), x, H, d)),
    "qkv_k_v_swapped": ("qkv_project", lambda x, w, H, d: _qkv_swapped(x, w, H, d)),
    "qkv_heads_interleaved": ("qkv_project", lambda x, w, H, d: _qkv_interleaved(x, w, H, d)),
    "merge_unweighted": (
        "merge_partials",
        lambda o, l: (np.asarray(o).mean(axis=0), np.logaddexp.reduce(np.asarray(l), axis=0)),
    ),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    owner = O
    if "." in attr:
        cls, attr = attr.split(".")
        owner = getattr(O, cls)
    monkeypatch.setattr(owner, attr, fn)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check()
        except (AssertionError, ValueError, IndexError, KeyError, ZeroDivisionError):
            caught.append(check.__name__)
    assert caught, f"no pin caught the planted mistake {name}"


def test_unmutated_oracle_passes_every_pin():
    for check in pins.ALL_CHECKS:
        check()
