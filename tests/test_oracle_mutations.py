"""Plant plausible mistakes in the CPU oracle and show that some pin catches each.

Every mutant is a deliberately wrong copy of one oracle function, swapped in
with monkeypatch for the duration of one test (CPU only).
"""
import numpy as np
import pytest

import pins
from oracle import cache_ops as co
from oracle import formats as fm
from oracle import paged_attention as pa


def _attend_mutant(gqa="div", use_scale=True, out_operand="v", normalise="sum"):
    def attend(q, k, v, scale):
        hq, d = q.shape
        hkv = k.shape[0]
        group = hq // hkv
        out = np.zeros((hq, d))
        lse = np.full(hq, -np.inf)
        for h in range(hq):
            g = h // group if gqa == "div" else h % hkv
            s = k[g] @ q[h] * (scale if use_scale else 1.0)
            m = s.max()
            p = np.exp(s - m)
            denom = p.sum() if normalise == "sum" else p.max()
            src = v[g] if out_operand == "v" else k[g]
            out[h] = (p @ src) / denom
            lse[h] = m + np.log(p.sum())
        return out, lse
    return attend


def _gather_reversed_blocks(cache, block_table, ctx, kv_dtype, scales=None):
    n = pa.num_blocks_for(ctx)
    reversed_table = np.asarray(block_table[:n])[::-1]
    return _real_gather(cache, reversed_table, ctx, kv_dtype, scales)


def _gather_shifted_tokens(cache, block_table, ctx, kv_dtype, scales=None):
    full = _real_gather(cache, block_table, min(ctx + 1, len(block_table) * 16), kv_dtype, scales)
    return full[:, 1:ctx + 1, :] if full.shape[1] > ctx else full[:, :ctx, :]


def _gather_ignores_scales(cache, block_table, ctx, kv_dtype, scales=None):
    return _real_gather(cache, block_table, ctx, kv_dtype, None)


_real_gather = pa.gather_kv


def _merge_plain_average(m, l, acc):
    live = np.isfinite(m)
    return (acc[live] / l[live][:, None]).mean(axis=0)


def _merge_no_rescale(m, l, acc):
    live = np.isfinite(m)
    return acc[live].sum(axis=0) / l[live].sum()


def _e4m3_value_bias8(code):
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp, man = (code >> 3) & 0xF, code & 7
    if exp == 15 and man == 7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -10
    return sign * (1 + man / 8) * 2.0 ** (exp - 8)


_real_encode = fm.e4m3_encode


def _encode_ties_away(x):
    x = np.asarray(x, dtype=np.float32)
    # nudge exact ties away from zero before the real (half-to-even) rounding
    a = np.abs(x).astype(np.float64)
    _, k = np.frexp(a)
    e = np.maximum(k - 1, -6)
    quantum = np.ldexp(1.0, e - 3)
    frac = a / quantum - np.floor(a / quantum)
    tie = frac == 0.5
    bumped = np.where(tie, a + quantum / 4, a) * np.sign(np.where(x == 0, 1.0, x))
    return _real_encode(bumped.astype(np.float32))


def _encode_truncating(x):
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    _, k = np.frexp(a)
    e = np.maximum(k - 1, -6)
    quantum = np.ldexp(1.0, e - 3)
    y = np.floor(a / quantum) * quantum
    return _real_encode((y * np.sign(np.where(x == 0, 1.0, x))).astype(np.float32))


def _bf16_wrong_shift(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)


_real_cache_write = co.cache_write_ref


def _cache_write_wrong_offset(k_cache, v_cache, new_k, new_v, slot_mapping, src_dtype, cache_dtype,
                              k_scale=None, v_scale=None):
    slots = np.asarray(slot_mapping, dtype=np.int64)
    shifted = np.where(slots >= 0, (slots // 16) * 16 + (slots + 1) % 16, slots)
    return _real_cache_write(k_cache, v_cache, new_k, new_v, shifted, src_dtype, cache_dtype,
                             k_scale, v_scale)


_real_copy = co.copy_blocks_ref


def _copy_blocks_swapped(k_cache, v_cache, pairs, k_scale=None, v_scale=None):
    p = np.asarray(pairs).reshape(-1, 2)[:, ::-1]
    return _real_copy(k_cache, v_cache, p, k_scale, v_scale)


def _positions_off_by_one(ctx, q_len):
    return np.arange(ctx - q_len, ctx, dtype=np.int64) - 1


def _positions_top_left(ctx, q_len):
    return np.arange(0, q_len, dtype=np.int64)


def _positions_no_causal_mask(ctx, q_len):
    return np.full(q_len, ctx - 1, dtype=np.int64)


_real_unpack = fm.int4_unpack


def _unpack_high_first(packed):
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b >> 4
    out[..., 1::2] = b & 0x0F
    return out


def _int4_offset_7(packed):
    return _real_unpack(packed).astype(np.float64) - 7


def _int4_encode_truncating(x):
    t = np.trunc(np.asarray(x, dtype=np.float32).astype(np.float64))
    return (np.clip(t, -8, 7) + 8).astype(np.uint8)


_real_int4_encode = fm.int4_encode


def _int4_encode_nan_to_zero(x):
    x = np.asarray(x, dtype=np.float32)
    codes = _real_int4_encode(x)
    return np.where(np.isnan(x), np.uint8(8), codes).astype(np.uint8)


MUTANTS = {
    "gqa_modulo_mapping": (pa, "attend", _attend_mutant(gqa="mod")),
    "scale_dropped": (pa, "attend", _attend_mutant(use_scale=False)),
    "k_instead_of_v": (pa, "attend", _attend_mutant(out_operand="k")),
    "normalised_by_max": (pa, "attend", _attend_mutant(normalise="max")),
    "block_order_reversed": (pa, "gather_kv", _gather_reversed_blocks),
    "token_offset_by_one": (pa, "gather_kv", _gather_shifted_tokens),
    "fp8_scale_ignored": (pa, "gather_kv", _gather_ignores_scales),
    "merge_plain_average": (pa, "lse_merge_ref", _merge_plain_average),
    "merge_without_rescale": (pa, "lse_merge_ref", _merge_no_rescale),
    "e4m3_bias_8": (fm, "e4m3_value", _e4m3_value_bias8),
    "e4m3_ties_away": (fm, "e4m3_encode", _encode_ties_away),
    "e4m3_truncating": (fm, "e4m3_encode", _encode_truncating),
    "bf16_wrong_shift": (fm, "bf16_to_f64", _bf16_wrong_shift),
    "cache_write_wrong_offset": (co, "cache_write_ref", _cache_write_wrong_offset),
    "copy_direction_swapped": (co, "copy_blocks_ref", _copy_blocks_swapped),
    "query_position_off_by_one": (pa, "query_positions", _positions_off_by_one),
    "causal_mask_top_left": (pa, "query_positions", _positions_top_left),
    "causal_mask_missing": (pa, "query_positions", _positions_no_causal_mask),
    "int4_nibble_order": (fm, "int4_unpack", _unpack_high_first),
    "int4_offset_7": (fm, "int4_to_f64", _int4_offset_7),
    "int4_truncating": (fm, "int4_encode", _int4_encode_truncating),
    "int4_nan_to_zero": (fm, "int4_encode", _int4_encode_nan_to_zero),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(name, monkeypatch):
    module, attr, mutant = MUTANTS[name]
    monkeypatch.setattr(module, attr, mutant)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check()
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
