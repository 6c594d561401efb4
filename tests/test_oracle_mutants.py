"""Planted mistakes in the oracle must each break at least one pin.

Every mutant replaces one step function of the oracle (on the CPU, for the
duration of one test) with a plausible bug: a dropped term, a wrong sign, a
wrong index or a transposed operand.  If the pin suite still passed, that
step would be unpinned.
"""

import math

import numpy as np
import pytest

import oracle
import oracle.decode_ref as ref
from oracle_pins import ALL_PINS


def _scores_noscale(q, keys, scale):
    return keys @ q


def _scores_negated(q, keys, scale):
    return -scale * (keys @ q)


def _attend_nomax(q, keys, values, scale):
    n = keys.shape[0]
    if n == 0:
        return np.zeros(values.shape[1]), -np.inf
    s = ref.scores(q, keys, scale)
    p = np.exp(s)
    return (p @ values) / np.sum(p), np.log(np.sum(p))


def _attend_log2(q, keys, values, scale):
    n = keys.shape[0]
    if n == 0:
        return np.zeros(values.shape[1]), -np.inf
    s = ref.scores(q, keys, scale)
    m = np.max(s)
    p = np.exp(s - m)
    return (p @ values) / np.sum(p), m + np.log2(np.sum(p))


def _attend_lse_nom(q, keys, values, scale):
    n = keys.shape[0]
    if n == 0:
        return np.zeros(values.shape[1]), -np.inf
    s = ref.scores(q, keys, scale)
    m = np.max(s)
    p = np.exp(s - m)
    return (p @ values) / np.sum(p), np.log(np.sum(p))


def _attend_mean_norm(q, keys, values, scale):
    n = keys.shape[0]
    if n == 0:
        return np.zeros(values.shape[1]), -np.inf
    s = ref.scores(q, keys, scale)
    m = np.max(s)
    p = np.exp(s - m)
    return (p @ values) / n, m + np.log(np.sum(p))


def _attend_drop_last(q, keys, values, scale):
    return ref.__dict__["_orig_attend"](q, keys[:-1], values[:-1], scale) if keys.shape[0] > 1 \
        else ref.__dict__["_orig_attend"](q, keys, values, scale)


def _token_locations_swapped(bt_row, ctx, bs):
    i = np.arange(ctx, dtype=np.int64)
    return np.asarray(bt_row, dtype=np.int64)[i % bs], i // bs


def _token_locations_reversed_slot(bt_row, ctx, bs):
    i = np.arange(ctx, dtype=np.int64)
    return np.asarray(bt_row, dtype=np.int64)[i // bs], (bs - 1 - i % bs)


def _token_locations_off_by_one(bt_row, ctx, bs):
    i = np.arange(1, ctx + 1, dtype=np.int64) if ctx else np.arange(0, dtype=np.int64)
    i = np.minimum(i, len(bt_row) * bs - 1)
    return np.asarray(bt_row, dtype=np.int64)[i // bs], i % bs


def _gather_kv_vtrans(k_pool, v_pool, pages, slots):
    k = k_pool[pages, :, slots, :]
    bs = v_pool.shape[3]
    dv = v_pool.shape[2]
    # reads V as if stored [bs][Dv] inside the (page, head) tile
    flat = v_pool.reshape(v_pool.shape[0], v_pool.shape[1], -1)
    idx = slots[:, None] * dv + np.arange(dv)[None, :]
    v = np.stack([flat[p, :, ix] for p, ix in zip(pages, idx)]) if len(pages) else \
        np.zeros((0, v_pool.shape[1], dv))
    return k, v


def _gather_kv_khead_swapped(k_pool, v_pool, pages, slots):
    k, v = ref.__dict__["_orig_gather_kv"](k_pool, v_pool, pages, slots)
    return k[:, ::-1, :], v


def _kv_head_mod(h, hq, hkv):
    return h % hkv


def _latent_kv_tail(c, dv):
    return c, c[:, c.shape[1] - dv:]


def _latent_kv_truncated_keys(c, dv):
    return c[:, :dv], c[:, :dv]


def _bf16_shift15(bits):
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    return u.view(np.float32).astype(np.float64)


def _bf16_as_fp16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _merge_unnormalised(o_parts, lse_parts):
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    big = np.max(lse_parts)
    if not np.isfinite(big):
        return np.zeros(o_parts.shape[1]), -np.inf
    w = np.exp(lse_parts - big)
    return w @ o_parts, big + np.log(np.sum(w))


def _merge_plain_mean(o_parts, lse_parts):
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    keep = np.isfinite(lse_parts)
    if not keep.any():
        return np.zeros(o_parts.shape[1]), -np.inf
    big = np.max(lse_parts)
    return o_parts[keep].mean(axis=0), big + np.log(np.sum(np.exp(lse_parts - big)))


def _chunk_alpha_flipped(q, keys, values, scale, bs, tok0):
    n = keys.shape[0]
    if n == 0:
        return np.zeros(values.shape[1]), -np.inf
    m, l, acc, start = -np.inf, 0.0, np.zeros(values.shape[1]), 0
    while start < n:
        end = min(n, start + bs - ((tok0 + start) % bs))
        s = ref.scores(q, keys[start:end], scale)
        m_new = max(m, float(np.max(s)))
        alpha = np.exp(m_new - m) if np.isfinite(m) else 0.0
        p = np.exp(s - m_new)
        l = alpha * l + np.sum(p)
        acc = alpha * acc + p @ values[start:end]
        m, start = m_new, end
    return acc / l, m + np.log(l)


def _chunk_l_not_rescaled(q, keys, values, scale, bs, tok0):
    n = keys.shape[0]
    if n == 0:
        return np.zeros(values.shape[1]), -np.inf
    m, l, acc, start = -np.inf, 0.0, np.zeros(values.shape[1]), 0
    while start < n:
        end = min(n, start + bs - ((tok0 + start) % bs))
        s = ref.scores(q, keys[start:end], scale)
        m_new = max(m, float(np.max(s)))
        alpha = np.exp(m - m_new) if np.isfinite(m) else 0.0
        p = np.exp(s - m_new)
        l = l + np.sum(p)
        acc = alpha * acc + p @ values[start:end]
        m, start = m_new, end
    return acc / l, m + np.log(l)


def _split_ranges_overlap(num_pages, c, ns):
    return [(min(num_pages, max(0, s * c - 1)), min(num_pages, (s + 1) * c)) for s in range(ns)]


def _split_ranges_gap(num_pages, c, ns):
    return [(min(num_pages, s * c + (1 if s else 0)), min(num_pages, (s + 1) * c)) for s in range(ns)]


def _append_slot_off_by_one(bt_row, n, bs):
    if n < 0 or n >= len(bt_row) * bs or bt_row[n // bs] < 0:
        return None
    return int(bt_row[n // bs]), (n + 1) % bs


def _append_slot_previous_page(bt_row, n, bs):
    if n < 0 or n >= len(bt_row) * bs or bt_row[n // bs] < 0:
        return None
    return int(bt_row[max(0, n // bs - 1)]), n % bs


def _append_slot_no_table_check(bt_row, n, bs):
    if n < 0 or n >= len(bt_row) * bs:
        return None
    return int(bt_row[n // bs]), n % bs


def _append_kv_skips_last(k_pool, v_pool, bt, ctx, k_new, v_new):
    return ref._orig_append_kv(k_pool, v_pool, bt[:-1], ctx[:-1], k_new[:-1], v_new[:-1])


def _row_context_off_by_one(ctx, q_len, j):
    return max(0, int(ctx) - q_len + j)


def _row_context_no_mask(ctx, q_len, j):
    return int(ctx)


def _row_context_reversed(ctx, q_len, j):
    return max(0, int(ctx) - j)


def _row_context_one_past(ctx, q_len, j):
    return min(int(ctx), max(0, int(ctx) - q_len + 2 + j))


def _fp8_bias8(bits):
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    mag = np.where(e == 0, m * 2.0 ** -10, (8 + m) * np.exp2(e - 11.0))
    v = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, v)


def _fp8_no_subnormals(bits):
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    mag = (8 + m) * np.exp2(e - 10.0)
    v = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, v)


def _fp8_unsigned(bits):
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    e, m = (b >> 3) & 15, b & 7
    v = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    return np.where((e == 15) & (m == 7), np.nan, v)


def _decode_scales_swapped(*a, k_scale=1.0, v_scale=1.0, **kw):
    return ref._orig_paged_decode(*a, k_scale=v_scale, v_scale=k_scale, **kw)


def _decode_v_unscaled(*a, k_scale=1.0, v_scale=1.0, **kw):
    return ref._orig_paged_decode(*a, k_scale=k_scale, v_scale=1.0, **kw)


def _mla_scales_swapped(*a, k_scale=1.0, v_scale=1.0, **kw):
    return ref._orig_paged_decode_mla(*a, k_scale=v_scale, v_scale=k_scale, **kw)


def _mla_k_scale_dropped(*a, k_scale=1.0, v_scale=1.0, **kw):
    return ref._orig_paged_decode_mla(*a, k_scale=1.0, v_scale=v_scale, **kw)


MUTANTS = {
    "scores_noscale": ("scores", _scores_noscale),
    "scores_negated": ("scores", _scores_negated),
    "attend_nomax": ("attend", _attend_nomax),
    "attend_log2": ("attend", _attend_log2),
    "attend_lse_without_max": ("attend", _attend_lse_nom),
    "attend_divide_by_count": ("attend", _attend_mean_norm),
    "attend_drops_last_token": ("attend", _attend_drop_last),
    "token_page_slot_swapped": ("token_locations", _token_locations_swapped),
    "token_slot_reversed": ("token_locations", _token_locations_reversed_slot),
    "token_off_by_one": ("token_locations", _token_locations_off_by_one),
    "v_read_transposed": ("gather_kv", _gather_kv_vtrans),
    "k_heads_reversed": ("gather_kv", _gather_kv_khead_swapped),
    "gqa_head_modulo": ("kv_head_of", _kv_head_mod),
    "mla_values_from_tail": ("latent_kv", _latent_kv_tail),
    "mla_keys_truncated": ("latent_kv", _latent_kv_truncated_keys),
    "bf16_shift_15": ("bf16_bits_to_f64", _bf16_shift15),
    "bf16_read_as_fp16": ("bf16_bits_to_f64", _bf16_as_fp16),
    "merge_unnormalised": ("merge_partials", _merge_unnormalised),
    "merge_plain_mean": ("merge_partials", _merge_plain_mean),
    "chunk_alpha_flipped": ("chunk_partial", _chunk_alpha_flipped),
    "chunk_l_not_rescaled": ("chunk_partial", _chunk_l_not_rescaled),
    "split_ranges_overlap": ("split_page_ranges", _split_ranges_overlap),
    "split_ranges_gap": ("split_page_ranges", _split_ranges_gap),
    "append_slot_off_by_one": ("append_slot", _append_slot_off_by_one),
    "append_slot_previous_page": ("append_slot", _append_slot_previous_page),
    "append_slot_no_table_check": ("append_slot", _append_slot_no_table_check),
    "append_kv_skips_last_sequence": ("append_kv", _append_kv_skips_last),
    "rows_context_off_by_one": ("row_context", _row_context_off_by_one),
    "rows_unmasked": ("row_context", _row_context_no_mask),
    "rows_reversed": ("row_context", _row_context_reversed),
    "rows_see_one_ahead": ("row_context", _row_context_one_past),
    "fp8_exponent_bias_8": ("fp8_e4m3_bits_to_f64", _fp8_bias8),
    "fp8_no_subnormals": ("fp8_e4m3_bits_to_f64", _fp8_no_subnormals),
    "fp8_sign_dropped": ("fp8_e4m3_bits_to_f64", _fp8_unsigned),
    "fp8_scales_swapped": ("paged_decode", _decode_scales_swapped),
    "fp8_v_scale_dropped": ("paged_decode", _decode_v_unscaled),
    "mla_fp8_scales_swapped": ("paged_decode_mla", _mla_scales_swapped),
    "mla_fp8_k_scale_dropped": ("paged_decode_mla", _mla_k_scale_dropped),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(ref.__dict__, "_orig_attend", ref.attend)
    monkeypatch.setitem(ref.__dict__, "_orig_gather_kv", ref.gather_kv)
    monkeypatch.setitem(ref.__dict__, "_orig_append_kv", ref.append_kv)
    monkeypatch.setitem(ref.__dict__, "_orig_paged_decode", ref.paged_decode)
    monkeypatch.setitem(ref.__dict__, "_orig_paged_decode_mla", ref.paged_decode_mla)
    monkeypatch.setattr(ref, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(ref)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant {name} passed every pin"
