"""Pins of oracle.cache_write_autoscale_ref (slot scatter that sets the block
scales itself): a whole-block write equals the plain scatter with the scale
amax/top; appends that fit equal the plain scatter with the block's scale;
a growing append sets the scale to exactly float32(amax/top) and re-encodes
every stored code as encode(value * old / new), both recomputed with torch's
float32 arithmetic and casts; it clips nothing and moves no stored value by
more than one new quantum; planted mistakes are caught."""
import numpy as np
import pytest
import torch

import oracle
from oracle import cache_ops as co

BLOCK = 16


def _f32(shape, rng, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def _values(cache, scales, kv):
    vals = oracle.e4m3_to_f64(cache) if kv == "fp8" else oracle.int4_to_f64(cache)
    return vals * scales.astype(np.float64)[:, :, None, None]


def _torch_scale(amax, top):
    """float32(amax / top) with torch's float32 division."""
    return (torch.from_numpy(np.asarray(amax, np.float32)) / torch.tensor(top, dtype=torch.float32)).numpy()


def _torch_reencode(codes, old, new, kv):
    """Codes of float32(float32(v * old) / new) for stored codes' values v:
    torch's float8_e4m3fn cast after saturation, or round-half-even and clamp
    for int4 (packed two per byte, element 2i in the low nibble)."""
    c = torch.from_numpy(np.ascontiguousarray(codes))
    if kv == "fp8":
        v = c.view(torch.float8_e4m3fn).to(torch.float32)
    else:
        lo, hi = (c & 15).to(torch.float32) - 8, (c >> 4).to(torch.float32) - 8
        v = torch.stack([lo, hi], dim=-1).reshape(c.shape[:-1] + (2 * c.shape[-1],))
    x = (v * torch.tensor(np.float32(old))) / torch.tensor(np.float32(new))
    if kv == "fp8":
        return x.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    q = (torch.round(x).clamp(-8, 7) + 8).to(torch.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).numpy()


def _empty_pool(nb, hkv, d, kv):
    width = d if kv == "fp8" else d // 2
    return np.zeros((nb, hkv, BLOCK, width), np.uint8), np.ones((nb, hkv), np.float32)


@pytest.mark.parametrize("kv", ["fp8", "int4"])
def test_whole_block_write_equals_plain_scatter(kv):
    rng = np.random.default_rng(161)
    hkv, d = 2, 128
    top = np.float32(448.0 if kv == "fp8" else 7.0)
    kc, ks = _empty_pool(4, hkv, d, kv)
    vc, vs = _empty_pool(4, hkv, d, kv)
    nk, nv = _f32((16, hkv, d), rng), _f32((16, hkv, d), rng, 3.0)
    slots = np.arange(16) + 2 * BLOCK
    k2, v2, ks2, vs2 = oracle.cache_write_autoscale_ref(kc, vc, ks, vs, nk, nv, slots, "f32", kv)
    want_ks = ks.copy()
    want_ks[2] = _torch_scale(np.abs(nk).max(axis=(0, 2)), top)
    assert np.array_equal(ks2.view(np.uint32), want_ks.view(np.uint32))
    kp, _ = oracle.cache_write_ref(kc, vc, nk, nv, slots, "f32", kv, want_ks, vs2)
    assert np.array_equal(k2, kp)


@pytest.mark.parametrize("kv", ["fp8", "int4"])
def test_appends_grow_the_scale_and_reencode(kv):
    rng = np.random.default_rng(162)
    hkv, d = 2, 128
    top = 448.0 if kv == "fp8" else 7.0
    kc, ks = _empty_pool(3, hkv, d, kv)
    vc, vs = _empty_pool(3, hkv, d, kv)
    # prompt of 5 tokens into block 1, then appends that fit and appends that grow
    rows = [_f32((5, hkv, d), rng)] + [_f32((1, hkv, d), rng, m) for m in (0.5, 4.0, 1.0, 9.0)]
    pos = 0
    for r in rows:
        n = r.shape[0]
        slots = BLOCK + pos + np.arange(n)
        before = _values(kc, ks, kv)[1, :, :pos]
        old_scale = ks[1].copy()
        kc2, vc2, ks2, vs2 = oracle.cache_write_autoscale_ref(kc, vc, ks, vs, r, r, slots, "f32", kv)
        a = np.abs(r).max(axis=(0, 2))
        grew = (a > old_scale * np.float32(top)) & (pos > 0)
        # the scale covers every new value: nothing is clipped
        assert np.all(ks2[1] * np.float32(top) >= a * (1 - 1e-6))
        # a scale that did not need to grow stayed
        assert np.array_equal(ks2[1][~grew & (pos > 0)], old_scale[~grew & (pos > 0)])
        # a grown scale is exactly float32(amax / top), and every stored code
        # is re-encoded from its value at the old scale
        for h in np.flatnonzero(grew):
            assert ks2[1, h].view(np.uint32) == _torch_scale(a[h], top).view(np.uint32)
            want = _torch_reencode(kc[1, h, :pos], old_scale[h], ks2[1, h], kv)
            assert np.array_equal(kc2[1, h, :pos], want)
        # stored values moved by at most one quantum of the new scale
        after = _values(kc2, ks2, kv)[1, :, :pos]
        quantum = ks2[1].astype(np.float64)[:, None, None] * (1.0 if kv == "int4" else 32.0)
        assert np.all(np.abs(after - before) <= quantum + 1e-12)
        # the new rows are encoded with the block's final scale, as the plain scatter does
        kp, _ = oracle.cache_write_ref(kc2, vc2, r, r, slots, "f32", kv, ks2, vs2)
        assert np.array_equal(kp, kc2)
        kc, vc, ks, vs = kc2, vc2, ks2, vs2
        pos += n
    assert pos == 9


class _NoReencode:
    def __init__(self):
        self.real = co.cache_write_autoscale_ref

    def __call__(self, k_cache, v_cache, k_scale, v_scale, new_k, new_v, slot_mapping, src_dtype, cache_dtype):
        # grow the scales as the reference does but keep the old codes
        k2, v2, ks, vs = self.real(k_cache, v_cache, k_scale, v_scale, new_k, new_v, slot_mapping, src_dtype,
                                   cache_dtype)
        slots = np.asarray(slot_mapping)
        blk, o0 = int(slots[0]) // BLOCK, int(slots[0]) % BLOCK
        k2[blk, :, :o0] = k_cache[blk, :, :o0]
        v2[blk, :, :o0] = v_cache[blk, :, :o0]
        return k2, v2, ks, vs


def _grow_double(k_cache, v_cache, k_scale, v_scale, new_k, new_v, slot_mapping, src_dtype, cache_dtype):
    """A planted mistake: a growing append sets the scale to 2 * amax / top
    (room to spare), re-encoding consistently with that wrong scale."""
    top = np.float32(448.0 if cache_dtype == "fp8" else 7.0)
    q = oracle.e4m3_quantize if cache_dtype == "fp8" else oracle.int4_quantize
    dec = oracle.e4m3_to_f64 if cache_dtype == "fp8" else oracle.int4_to_f64
    outs = []
    for cache, scale, new in ((k_cache, k_scale, new_k), (v_cache, v_scale, new_v)):
        cache, scale = cache.copy(), scale.copy()
        slots = np.asarray(slot_mapping)
        blk, o0 = int(slots[0]) // BLOCK, int(slots[0]) % BLOCK
        rows = np.asarray(new, np.float32)
        for h in range(cache.shape[1]):
            a = np.float32(np.abs(rows[:, h]).max())
            s = scale[blk, h]
            if o0 == 0:
                s = np.float32(a / top)
            elif a > np.float32(scale[blk, h] * top):
                s = np.float32(2 * a / top)
                kept = dec(cache[blk, h, :o0]).astype(np.float32) * scale[blk, h]
                cache[blk, h, :o0] = q(kept, s)
            scale[blk, h] = s
            for i, slot in enumerate(slots):
                cache[blk, h, int(slot) % BLOCK] = q(rows[i, h], s)
        outs.append((cache, scale))
    return outs[0][0], outs[1][0], outs[0][1], outs[1][1]


def test_missing_reencode_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "cache_write_autoscale_ref", _NoReencode())
    with pytest.raises(AssertionError):
        test_appends_grow_the_scale_and_reencode("fp8")


@pytest.mark.parametrize("kv", ["fp8", "int4"])
def test_scale_grown_too_far_is_caught(kv, monkeypatch):
    monkeypatch.setattr(oracle, "cache_write_autoscale_ref", _grow_double)
    with pytest.raises(AssertionError):
        test_appends_grow_the_scale_and_reencode(kv)
