"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

Every mutation below is a slip one could make writing the oracle from the
pages: a dropped term, a wrong sign, index or offset, a transposed operand.
The pins in test_oracle_pins.py must turn at least one of them red.
"""
import math

import numpy as np
import pytest
import torch

import drafter_synth as ds
import oracle
import oracle.drafter_attn_oracle as mod
from tests import test_oracle_pins as pins
from tests.bruteforce import bruteforce

orig_rms = mod.rms_norm
orig_rope = mod.rope_neox
orig_freq = mod.rope_inv_freq
orig_gather = mod.gather_context
orig_attend = mod._softmax_attend
orig_qknr = mod.qk_norm_rope
orig_append = mod.kv_append
orig_paged = mod.paged_attn
orig_merge = mod._merge_parts


def _merge_no_rescale(parts, b, D):
    # every range weighted 1 instead of exp(m - M)
    return orig_merge([(np.where(np.isfinite(m), 0.0, m), l, o) for m, l, o in parts], b, D)


def _merge_max_of_first(parts, b, D):
    # the reference maximum taken from the first range only
    M0 = parts[0][0]
    return orig_merge([(np.minimum(m, M0) if i else m, l, o) for i, (m, l, o) in enumerate(parts)], b, D)


def _append_next_slot(k_pool, v_pool, qkv, page_table, context_lens, block_lens=None, **kw):
    return orig_append(k_pool, v_pool, qkv, page_table, np.asarray(context_lens) + 1, block_lens, **kw)


def _append_v_as_k(k_pool, v_pool, qkv, page_table, context_lens, block_lens=None, **kw):
    k, v = orig_append(k_pool, v_pool, qkv, page_table, context_lens, block_lens, **kw)
    _, v2 = orig_append(v_pool, v_pool, qkv, page_table, context_lens, block_lens, **kw)
    return np.where(k != np.asarray(k_pool), v2, k), v


def _paged_drop_last(qkv, k_pool, v_pool, page_table, kv_lens, block_lens=None, **kw):
    return orig_paged(qkv, k_pool, v_pool, page_table, np.maximum(np.asarray(kv_lens) - 1, 0), block_lens, **kw)


def _qknr_rotates_v(qkv, positions, qw, kw, *, num_q_heads, num_kv_heads, eps=1e-5, rope_base=1e4, yarn=None):
    x = orig_qknr(qkv, positions, qw, kw, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, eps=eps,
                  rope_base=rope_base)
    for g in range(num_kv_heads):
        c = mod.v_cols(g, num_q_heads, num_kv_heads)
        x[:, c] = orig_rope(orig_rms(x[:, c], kw, eps), positions, rope_base)
    return x


def _qknr_k_with_q_weight(qkv, positions, qw, kw, **kw2):
    return orig_qknr(qkv, positions, qw, qw, **kw2)


def _qknr_rope_then_norm(qkv, positions, qw, kw, *, num_q_heads, num_kv_heads, eps=1e-5, rope_base=1e4, yarn=None):
    x = np.array(qkv, dtype=np.float64, copy=True)
    pos = np.asarray(positions)
    for h in range(num_q_heads):
        c = mod.q_cols(h, num_q_heads, num_kv_heads)
        x[:, c] = orig_rms(orig_rope(x[:, c], pos, rope_base), qw, eps)
    for g in range(num_kv_heads):
        c = mod.k_cols(g, num_q_heads, num_kv_heads)
        x[:, c] = orig_rms(orig_rope(x[:, c], pos, rope_base), kw, eps)
    return x


def _qknr_skip_last_k(qkv, positions, qw, kw, *, num_q_heads, num_kv_heads, eps=1e-5, rope_base=1e4, yarn=None):
    x = orig_qknr(qkv, positions, qw, kw, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, eps=eps,
                  rope_base=rope_base)
    c = mod.k_cols(num_kv_heads - 1, num_q_heads, num_kv_heads)
    x[:, c] = np.asarray(qkv, dtype=np.float64)[:, c]
    return x


def _rope_sign(x, pos, base, yarn=None):
    if yarn is not None:
        return orig_rope(x, pos, base, yarn)
    x = np.asarray(x, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * orig_freq(base, x.shape[-1])
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :32], x[..., 32:]
    return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1)


def _rope_interleaved(x, pos, base, yarn=None):
    if yarn is not None:
        return orig_rope(x, pos, base, yarn)
    x = np.asarray(x, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * orig_freq(base, x.shape[-1])
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x1 * c - x2 * s
    y[..., 1::2] = x2 * c + x1 * s
    return y


orig_yfreq = mod.yarn_inv_freq
orig_mscale = mod.yarn_mscale


orig_pair = mod.yarn_pair_at_turns


def _yarn_ramp_reversed(base, factor, L, alpha=1.0, beta=32.0, dim=64, ramp="turns"):
    if ramp != "turns":
        return orig_yfreq(base, factor, L, alpha, beta, dim, ramp)
    theta = orig_freq(base, dim)
    g = np.clip((beta - L * theta / (2 * np.pi)) / (beta - alpha), 0.0, 1.0)
    return (1 - g) * theta / factor + g * theta


def _yarn_turns_without_2pi(base, factor, L, alpha=1.0, beta=32.0, dim=64, ramp="turns"):
    if ramp != "turns":
        return orig_yfreq(base, factor, L, alpha, beta, dim, ramp)
    return orig_yfreq(base, factor, L * 2 * np.pi, alpha, beta, dim)


def _yarn_times_s(base, factor, L, alpha=1.0, beta=32.0, dim=64, ramp="turns"):
    return orig_yfreq(base, 1.0 / factor, L, alpha, beta, dim, ramp)


def _index_ramp(base, factor, L, alpha, beta, dim, round_lo, round_hi, inverted=False):
    theta = orig_freq(base, dim)
    lo = round_lo(min(max(orig_pair(base, L, beta, dim), 0.0), dim / 2 - 1))
    hi = round_hi(min(max(orig_pair(base, L, alpha, dim), 0.0), dim / 2 - 1))
    i = np.arange(dim // 2)
    ramp = np.clip((i - lo) / (hi - lo), 0.0, 1.0) if hi > lo else (i > lo).astype(float)
    g = ramp if inverted else 1.0 - ramp
    return (1 - g) * theta / factor + g * theta


def _yarn_index_rounding_swapped(base, factor, L, alpha=1.0, beta=32.0, dim=64, ramp="turns"):
    if ramp != "index":
        return orig_yfreq(base, factor, L, alpha, beta, dim, ramp)
    return _index_ramp(base, factor, L, alpha, beta, dim, math.ceil, math.floor)


def _yarn_index_ramp_inverted(base, factor, L, alpha=1.0, beta=32.0, dim=64, ramp="turns"):
    if ramp == "turns":
        return orig_yfreq(base, factor, L, alpha, beta, dim, ramp)
    rnd = (math.floor, math.ceil) if ramp == "index" else (float, float)
    return _index_ramp(base, factor, L, alpha, beta, dim, *rnd, inverted=True)


def _rope_ignores_mscale(x, pos, base, yarn=None):
    return orig_rope(x, pos, base, None if yarn is None else {k: v for k, v in yarn.items() if k != "mscale"})


def _gather_shift_slot(k_pool, v_pool, row, L, g):
    k, v = orig_gather(k_pool, v_pool, row, L, g)
    return np.roll(k, 1, axis=0), v


def _gather_next_entry(k_pool, v_pool, row, L, g):
    if row is None:
        return orig_gather(k_pool, v_pool, row, L, g)
    return orig_gather(k_pool, v_pool, np.roll(np.asarray(row), -1) % k_pool.shape[0], L, g)


def _gather_full_pages_only(k_pool, v_pool, row, L, g):
    return orig_gather(k_pool, v_pool, row, (L // 64) * 64, g)


def _gather_other_head(k_pool, v_pool, row, L, g):
    return orig_gather(k_pool, v_pool, row, L, (g + 1) % k_pool.shape[1])


def _attend_no_scale(q, keys, vals, scale):
    return orig_attend(q, keys, vals, 1.0)


def _attend_wrong_axis(q, keys, vals, scale):
    s = scale * (q @ keys.T)
    e = np.exp(s - s.max())
    p = e / e.sum(axis=0, keepdims=True)
    return p @ vals, p


def _attend_context_only(q, keys, vals, scale):
    n = max(1, keys.shape[0] - q.shape[0])
    return orig_attend(q, keys[:n], vals[:n], scale)


def _attend_v_is_k(q, keys, vals, scale):
    return orig_attend(q, keys, keys, scale)


MUTATIONS = {
    "rms_no_eps": ("rms_norm", lambda x, w, eps: orig_rms(x, w, 0.0)),
    "rms_sum_not_mean": ("rms_norm", lambda x, w, eps: np.asarray(x) * w / np.sqrt(np.sum(np.asarray(x) ** 2, -1, keepdims=True) + eps)),
    "rms_one_plus_w": ("rms_norm", lambda x, w, eps: orig_rms(x, 1.0 + np.asarray(w), eps)),
    "rms_no_weight": ("rms_norm", lambda x, w, eps: orig_rms(x, np.ones_like(w), eps)),
    "rope_sign": ("rope_neox", _rope_sign),
    "rope_interleaved": ("rope_neox", _rope_interleaved),
    "rope_pos_plus_one": ("rope_neox", lambda x, pos, base, yarn=None: orig_rope(x, np.asarray(pos) + 1, base, yarn)),
    "rope_exponent": ("rope_inv_freq", lambda base, dim=64: np.power(float(base), -np.arange(dim // 2) / dim)),
    "rope_base_1000": ("rope_inv_freq", lambda base, dim=64: orig_freq(1000.0, dim)),
    "gather_slot_shift": ("gather_context", _gather_shift_slot),
    "gather_next_entry": ("gather_context", _gather_next_entry),
    "gather_drop_tail": ("gather_context", _gather_full_pages_only),
    "gather_other_head": ("gather_context", _gather_other_head),
    "gqa_modulo": ("kv_head_of", lambda h: h % 2),
    "k_from_v_cols": ("k_cols", lambda g, Hq, Hkv: mod.v_cols(g, Hq, Hkv)),
    "v_from_k_cols": ("v_cols", lambda g, Hq, Hkv: slice((Hq + g) * 64, (Hq + g + 1) * 64)),
    "q_head_offset": ("q_cols", lambda h, Hq, Hkv: slice(((h + 1) % Hq) * 64, ((h + 1) % Hq + 1) * 64)),
    "no_scale": ("_softmax_attend", _attend_no_scale),
    "softmax_wrong_axis": ("_softmax_attend", _attend_wrong_axis),
    "drop_block_keys": ("_softmax_attend", _attend_context_only),
    "values_are_keys": ("_softmax_attend", _attend_v_is_k),
    "qknr_rotates_v": ("qk_norm_rope", _qknr_rotates_v),
    "qknr_k_with_q_weight": ("qk_norm_rope", _qknr_k_with_q_weight),
    "qknr_rope_then_norm": ("qk_norm_rope", _qknr_rope_then_norm),
    "qknr_skip_last_k_head": ("qk_norm_rope", _qknr_skip_last_k),
    "append_next_slot": ("kv_append", _append_next_slot),
    "append_v_as_k": ("kv_append", _append_v_as_k),
    "paged_drops_last_key": ("paged_attn", _paged_drop_last),
    "yarn_ramp_reversed": ("yarn_inv_freq", _yarn_ramp_reversed),
    "yarn_turns_without_2pi": ("yarn_inv_freq", _yarn_turns_without_2pi),
    "yarn_multiplies_by_s": ("yarn_inv_freq", _yarn_times_s),
    "yarn_mscale_log10": ("yarn_mscale", lambda f: 0.1 * np.log10(f) + 1.0),
    "yarn_no_mscale": ("yarn_mscale", lambda f: 1.0),
    "yarn_index_rounding_swapped": ("yarn_inv_freq", _yarn_index_rounding_swapped),
    "yarn_index_ramp_inverted": ("yarn_inv_freq", _yarn_index_ramp_inverted),
    "yarn_pair_index_over_full_dim": ("yarn_pair_at_turns", lambda base, L, t, dim=64: orig_pair(base, L, t, 2 * dim)),
    "yarn_pair_index_without_2pi": ("yarn_pair_at_turns", lambda base, L, t, dim=64: orig_pair(base, L * 2 * math.pi, t, dim)),
    "yarn_explicit_mscale_ignored": ("rope_neox", _rope_ignores_mscale),
    "merge_no_rescale": ("_merge_parts", _merge_no_rescale),
    "merge_max_of_first_range": ("_merge_parts", _merge_max_of_first),
}


def _battery():
    """Run a cheap set of pins; return the names of those that failed."""
    failed = []
    cases = [
        ds.make_case(2, 3, 12, 2, [65, 130], seed=77, qknorm=True, pool_pages=6),
        ds.make_case(2, 2, 6, 1, [64, 3], seed=78, qknorm=False, pool_pages=4),
    ]
    for i, c in enumerate(cases):
        try:
            ref = bruteforce(**c.np_args(), qknorm=c.qknorm)
            got = pins._oracle(c)
            if not pins._rel(got, ref) <= pins.TOL:
                failed.append(f"bruteforce{i}")
        except Exception:  # any error is a failed pin
            failed.append(f"bruteforce{i}")
    for name in ("test_rmsnorm_closed_forms", "test_rope_closed_forms", "test_qk_norm_rope_closed_forms",
                 "test_qk_norm_rope_constant_heads_at_position_zero", "test_yarn_factor_one_is_plain_rope",
                 "test_yarn_short_original_context_is_position_interpolation",
                 "test_yarn_long_original_context_only_scales", "test_yarn_ramp_midpoint_and_shape",
                 "test_yarn_ramps_agree_outside_the_ramp", "test_yarn_index_ramp_degenerate_bounds",
                 "test_yarn_index_ramp_factor_one_and_explicit_mscale"):
        try:
            getattr(pins, name)()
        except Exception:  # any error is a failed pin
            failed.append(name)
    for name in ("test_yarn_index_ramp_bounds_from_turn_counts", "test_yarn_unrounded_index_ramp"):
        try:
            getattr(pins, name)(*pins.YARN_INDEX_CASES[0])
        except Exception:  # any error is a failed pin
            failed.append(name)
    for i in (0, 1):
        try:
            pins.test_replaced_path_equals_fused_definition(i)
        except Exception:  # any error is a failed pin
            failed.append(f"replaced{i}")
    # the split-merge algebra, flat and in two levels, on a small case
    sm = ds.make_case(2, 3, 12, 2, [700, 130], seed=79, qknorm=True, pool_pages=14)
    for S, G in ((3, None), (9, 4)):
        try:
            got = oracle.drafter_attn_split_merge(**sm.np_args(), num_splits=S, group=G, qknorm=True)
            if not pins._rel(got, pins._oracle(sm)) <= pins.TOL:
                failed.append(f"split_merge{S}")
        except Exception:  # any error is a failed pin
            failed.append(f"split_merge{S}")
    for where in ("first", "tail_slot", "block"):
        try:
            pins.test_needle(where)
        except Exception:  # any error is a failed pin
            failed.append(f"needle_{where}")
    return failed


def test_battery_green_on_unmutated_oracle():
    assert _battery() == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    assert _battery(), f"no pin caught mutation {name}"
