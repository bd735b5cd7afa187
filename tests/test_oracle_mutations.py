"""Plant plausible mistakes in the oracle (CPU only) and check a pin catches each.

This shows the pins are strong enough: a dropped term, a wrong sign, a wrong
index or a transposed operand anywhere in the oracle fails at least one of
them. The oracle itself is restored after every case by ``monkeypatch``.
"""

import numpy as np
import pytest

import oracle_pins
from oracle import attn64, norm64, pool64, rope64, tiers64


def _rotate_with(fn):
    def rotate(x, phi):
        x = np.asarray(x, dtype=np.float64)
        squeeze = x.ndim == 2
        if squeeze:
            x = x[:, None, :]
        n, _, d = x.shape
        phi = np.asarray(phi, dtype=np.float64).reshape(n, d // 2)
        out = fn(x, np.cos(phi)[:, None, :], np.sin(phi)[:, None, :])
        return out[:, 0, :] if squeeze else out
    return rotate


def _adjacent(form):
    def fn(x, c, s):
        out = np.empty_like(x)
        xe, xo = x[..., 0::2], x[..., 1::2]
        out[..., 0::2], out[..., 1::2] = form(xe, xo, c, s)
        return out
    return fn


def _half_split(x, c, s):
    half = x.shape[-1] // 2
    out = np.empty_like(x)
    a, b = x[..., :half], x[..., half:]
    out[..., :half] = a * c - b * s
    out[..., half:] = a * s + b * c
    return out


def _freq_with(expo):
    def pair_axis_and_freq(axis_dims, theta):
        axis, freq = [], []
        for a, width in enumerate(axis_dims):
            for i in range(int(width) // 2):
                axis.append(a)
                freq.append(float(theta) ** expo(i, int(width), sum(axis_dims)))
        return np.asarray(axis), np.asarray(freq)
    return pair_axis_and_freq


def _angles_reversed_axes(pos, axis_dims, theta):
    pos = np.asarray(pos, dtype=np.float64).reshape(-1, 3)
    axis, freq = rope64.pair_axis_and_freq(axis_dims, theta)
    return pos[:, 2 - axis] * freq[None, :]


def _attention_with(weighted, softmax_axis=-1, use_scale=True):
    def attention(q, k, v, scale, block=512):
        q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
        out = np.empty(q.shape, dtype=np.float64)
        for h in range(q.shape[1]):
            s = (scale if use_scale else 1.0) * (q[:, h, :] @ k[:, h, :].T)
            m = np.max(s, axis=softmax_axis, keepdims=True)
            e = np.exp(s - m)
            p = e / np.sum(e, axis=softmax_axis, keepdims=True)
            out[:, h, :] = p @ weighted(k, v)[:, h, :]
        return out
    return attention


def _rotated_keys_unrotated(segments, axis_dims, theta, k_norm=None):
    ks = [np.asarray(k, dtype=np.float64) for k, _, _ in segments]
    vs = [np.asarray(v, dtype=np.float64) for _, v, _ in segments]
    return np.concatenate(ks), np.concatenate(vs)


def _rms_with(denom):
    def rmsnorm(x, weight, eps):
        x = np.asarray(x, dtype=np.float64)
        y = x / denom(x, float(eps))
        return y if weight is None else y * np.asarray(weight, dtype=np.float64)
    return rmsnorm


def _rms_weight_first(x, weight, eps):
    x = np.asarray(x, dtype=np.float64)
    if weight is not None:
        x = x * np.asarray(weight, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _prepare_rotate_first(x, pos, norm, axis_dims, theta):
    x = np.asarray(x, dtype=np.float64)
    if x.shape[0] == 0:
        return x
    if pos is not None:
        x = rope64.rotate(x, rope64.angles(pos, axis_dims, theta))
    if norm is not None:
        x = norm64.rmsnorm(x, norm[0], norm[1])
    return x


def _prepare_norm_ignored(x, pos, norm, axis_dims, theta):
    x = np.asarray(x, dtype=np.float64)
    if pos is not None and x.shape[0] > 0:
        x = rope64.rotate(x, rope64.angles(pos, axis_dims, theta))
    return x


def _pool_with(reduce, order_hw=True, swap_grid=False):
    def pool_frames(x, grid_h, grid_w, s):
        x = np.asarray(x, dtype=np.float64)
        if swap_grid:
            grid_h, grid_w = grid_w, grid_h
        frames = x.shape[0] // (grid_h * grid_w)
        rest = x.shape[1:]
        b = reduce(x.reshape((frames, grid_h // s, s, grid_w // s, s) + rest))
        if not order_hw:
            b = np.swapaxes(b, 1, 2)
        return b.reshape((frames * (grid_h // s) * (grid_w // s),) + rest)
    return pool_frames


def _split_with(lse_form, normalise=True):
    def split_attention(q, k, v, scale, key_ranges):
        q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
        nq, heads, d = q.shape
        partial = np.empty((len(key_ranges), nq, heads, d))
        lse = np.empty((len(key_ranges), nq, heads))
        for r, (a, b) in enumerate(key_ranges):
            for h in range(heads):
                sc = scale * (q[:, h, :] @ k[a:b, h, :].T)
                m = np.max(sc, axis=-1, keepdims=True)
                e = np.exp(sc - m)
                z = np.sum(e, axis=-1, keepdims=True)
                partial[r, :, h, :] = ((e / z) if normalise else e) @ v[a:b, h, :]
                lse[r, :, h] = lse_form(m, z)[:, 0]
        return partial, lse
    return split_attention


def _template_reversed(frames):
    names = [n for n, _, _ in tiers64.TIERS][::-1] + ["current"]
    return {n: list(range(1 + i * frames, 1 + (i + 1) * frames)) for i, n in enumerate(names)}


def _cell_corner(t_values, grid_h, grid_w, s):
    gh, gw = grid_h // s, grid_w // s
    hh, ww = np.meshgrid(np.arange(gh) * s, np.arange(gw) * s, indexing="ij")
    return np.concatenate([np.stack([np.full(gh * gw, float(t)), hh.reshape(-1), ww.reshape(-1)], axis=1)
                           for t in t_values], axis=0)


MUTATIONS = {
    "pool_sum_not_mean": [(pool64, "pool_frames", _pool_with(lambda b: b.sum(axis=(2, 4))))],
    "pool_first_cell_only": [(pool64, "pool_frames", _pool_with(lambda b: b[:, :, 0, :, 0]))],
    "pool_cells_column_major": [(pool64, "pool_frames", _pool_with(lambda b: b.mean(axis=(2, 4)), order_hw=False))],
    "pool_grid_transposed": [(pool64, "pool_frames", _pool_with(lambda b: b.mean(axis=(2, 4)), swap_grid=True))],
    "split_lse_log2": [(attn64, "split_attention", _split_with(lambda m, z: m + np.log2(z)))],
    "split_lse_no_max": [(attn64, "split_attention", _split_with(lambda m, z: np.log(z)))],
    "split_partial_unnormalised": [(attn64, "split_attention", _split_with(lambda m, z: m + np.log(z), False))],
    "rms_sum_not_mean": [(norm64, "rmsnorm", _rms_with(lambda x, e: np.sqrt(np.sum(x * x, -1, keepdims=True) + e)))],
    "rms_no_sqrt": [(norm64, "rmsnorm", _rms_with(lambda x, e: np.mean(x * x, -1, keepdims=True) + e))],
    "rms_eps_outside_sqrt": [(norm64, "rmsnorm", _rms_with(lambda x, e: np.sqrt(np.mean(x * x, -1, keepdims=True)) + e))],
    "rms_weight_before_norm": [(norm64, "rmsnorm", _rms_weight_first)],
    "norm_after_rotation": [(attn64, "prepare", _prepare_rotate_first)],
    "norm_ignored": [(attn64, "prepare", _prepare_norm_ignored)],
    "clockwise_turn": [(rope64, "rotate", _rotate_with(_adjacent(
        lambda xe, xo, c, s: (xe * c + xo * s, -xe * s + xo * c))))],
    "cos_sin_swapped": [(rope64, "rotate", _rotate_with(_adjacent(
        lambda xe, xo, c, s: (xe * s - xo * c, xe * c + xo * s))))],
    "half_split_pairs": [(rope64, "rotate", _rotate_with(_half_split))],
    "second_term_dropped": [(rope64, "rotate", _rotate_with(_adjacent(
        lambda xe, xo, c, s: (xe * c, xe * s + xo * c))))],
    "freq_missing_factor_2": [(rope64, "pair_axis_and_freq", _freq_with(lambda i, w, d: -1.0 * i / w))],
    "freq_over_head_dim": [(rope64, "pair_axis_and_freq", _freq_with(lambda i, w, d: -2.0 * i / d))],
    "freq_index_off_by_one": [(rope64, "pair_axis_and_freq", _freq_with(lambda i, w, d: -2.0 * (i + 1) / w))],
    "axes_reversed": [(rope64, "angles", _angles_reversed_axes)],
    "softmax_unnormalised": [(attn64, "softmax_rows", lambda s: np.exp(np.asarray(s) - np.max(s, axis=-1, keepdims=True)))],
    "softmax_over_queries": [(attn64, "attention", _attention_with(lambda k, v: v, softmax_axis=0))],
    "weights_times_keys": [(attn64, "attention", _attention_with(lambda k, v: k))],
    "scale_dropped": [(attn64, "attention", _attention_with(lambda k, v: v, use_scale=False))],
    "keys_not_rotated": [(attn64, "rotated_keys", _rotated_keys_unrotated)],
    # history tiers: ages swapped, one step late, the current chunk fed back as history,
    # the template's tier order reversed, a pooled cell at its corner instead of its centre
    "tier_ages_swapped": [(tiers64, "TIERS", (("pool4", 4, 2), ("pool2", 2, 3), ("prev", 1, 1)))],
    "tier_ages_late": [(tiers64, "TIERS", (("pool4", 4, 4), ("pool2", 2, 3), ("prev", 1, 2)))],
    "tier_prev_is_current": [(tiers64, "TIERS", (("pool4", 4, 3), ("pool2", 2, 2), ("prev", 1, 0)))],
    "tier_template_reversed": [(tiers64, "template_t", _template_reversed)],
    "tier_cell_corner": [(tiers64, "cell_positions", _cell_corner)],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    for module, attr, repl in MUTATIONS[name]:
        monkeypatch.setattr(module, attr, repl)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError, ZeroDivisionError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
