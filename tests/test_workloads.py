"""Layout invariants of the seeded workloads (host block manager, no attention math)."""
import math

import numpy as np
import pytest

import oracle
import pa_workloads as W


def _live_blocks(wl):
    return [list(wl.block_tables[b, :oracle.pages_for(int(c))]) for b, c in enumerate(wl.context_lens)]


def test_config1_shape_and_layout():
    wl = W.config1()
    assert wl.q.shape == (4, 4, 64) and wl.q.dtype == np.float32
    assert wl.k_cache.shape == (16, 4, 16, 64) and wl.k_cache.dtype == np.float32
    assert list(wl.context_lens) == [17, 33, 48, 5]
    assert wl.block_tables.shape == (4, 4) and wl.num_blocks == 16
    live = _live_blocks(wl)
    flat = [b for t in live for b in t]
    assert len(flat) == len(set(flat)) == 2 + 3 + 3 + 1
    assert math.isclose(wl.scale, 1 / 8)
    # padding points at an unused, NaN-filled block
    pad = wl.meta["pad_block"]
    assert pad not in flat and np.isnan(wl.k_cache[pad]).all()


def test_poison_marks_every_byte_decode_must_not_read():
    wl = W.config1()
    live = _live_blocks(wl)
    used = {b for t in live for b in t}
    for blk in range(wl.num_blocks):
        if blk not in used:
            assert np.isnan(wl.k_cache[blk]).all() and np.isnan(wl.v_cache[blk]).all()
    for b, c in enumerate(wl.context_lens):
        c = int(c)
        last = live[b][-1]
        tail = (c % 16) or 16
        assert np.isnan(wl.k_cache[last, :, tail:]).all()
        # the new token's slot is poisoned until the cache write
        s = int(wl.slot_mapping[b])
        assert s == live[b][(c - 1) // 16] * 16 + (c - 1) % 16
        assert np.isnan(wl.k_cache[s // 16, :, s % 16]).all()
        if c > 1:
            assert not np.isnan(wl.k_cache[live[b][0], :, 0]).any()


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_pool_sizes_and_tables(cfg):
    wl = W.CONFIGS[cfg](with_values=False)
    need = sum(oracle.pages_for(int(c)) for c in wl.context_lens)
    assert wl.num_blocks == math.ceil(1.1 * need)
    W.validate_tables(wl.block_tables, wl.context_lens, wl.num_blocks)
    W.validate_slots(wl.slot_mapping, wl.num_blocks)
    live = _live_blocks(wl)
    flat = np.concatenate([np.array(t) for t in live])
    assert np.unique(flat).size == flat.size == need
    # internal waste < one block per sequence (batching page, section 三)
    for c in wl.context_lens:
        assert oracle.internal_waste_tokens(int(c)) < 16


def test_config_shapes_match_the_workload_statements():
    c2 = W.config2(with_values=False)
    assert c2.num_seqs == 64 and (c2.num_q_heads, c2.num_kv_heads, c2.head_dim) == (32, 8, 128)
    assert c2.context_lens.min() >= 128 and c2.context_lens.max() <= 4096
    c3 = W.config3(with_values=False)
    assert c3.num_seqs == 256 and (c3.num_q_heads, c3.num_kv_heads) == (64, 8)
    assert c3.context_lens.min() >= 16 and c3.context_lens.max() <= 8192
    assert 1500 < np.median(c3.context_lens) < 2800
    c5 = W.config5(with_values=False)
    assert c5.num_seqs == 8 and set(c5.context_lens) == {131072} and c5.partition_tokens == 512
    assert c5.kv_dtype == "fp8" and c5.q_dtype == "bf16"


def test_shared_prefix_layout():
    wl = W.config4(with_values=False)
    P, S, npre = 32, 8, 125
    assert wl.num_seqs == P * S and wl.meta["prefix_blocks"] == npre
    shared = wl.block_tables_shared
    for p in range(P):
        rows = shared[p * S:(p + 1) * S, :npre]
        assert (rows == rows[0]).all()                       # every sample shares the prefix
        assert (wl.refcount[rows[0]] == S).all()             # refcount 8
    pairs = wl.copy_pairs
    assert pairs.shape == (P * S, 2)
    W.validate_copy_pairs(pairs, wl.num_blocks)
    for i in range(P * S):
        assert pairs[i, 0] == shared[i, npre - 1] and pairs[i, 1] == wl.block_tables[i, npre - 1]
        diff = np.flatnonzero(shared[i] != wl.block_tables[i])
        assert list(diff) == [npre - 1]
    assert (wl.context_lens >= 2001).all() and (wl.context_lens <= 2512).all()
    # suffix blocks are private
    suffix = [b for i in range(P * S) for b in wl.block_tables[i, npre:oracle.pages_for(int(wl.context_lens[i]))]]
    assert len(suffix) == len(set(suffix))


def test_shared_prefix_values_small():
    wl = W.make_shared_prefix_workload(name="t", seed=9, num_prompts=2, samples_per_prompt=3,
                                       prefix_tokens=48, suffix_max=20, num_q_heads=4,
                                       num_kv_heads=2, head_dim=16)
    # copy destinations start poisoned; the new-token slot is poisoned
    bits = wl.k_cache.view(np.uint16)
    for src, dst in wl.copy_pairs:
        assert (bits[dst] == 0x7FC0).all()
        assert not (bits[src] == 0x7FC0).all()


def test_fp8_values_mode_scales_cover_new_tokens():
    wl = W.make_workload(name="t", seed=3, context_lens=[20, 47], num_q_heads=8, num_kv_heads=2,
                         head_dim=16, q_dtype="bf16", kv_dtype="fp8", fp8_mode="values")
    assert wl.k_cache is None and wl.k_values is not None
    for t, s in enumerate(wl.slot_mapping):
        blk = s // 16
        x = oracle.bf16_to_f64(wl.new_k[t])
        assert (np.abs(x) <= wl.k_scale[blk][:, None] * 448 * (1 + 1e-6)).all()


def test_fp8_codes_mode_has_no_nan_in_live_blocks():
    wl = W.make_workload(name="t", seed=4, context_lens=[64, 33], num_q_heads=8, num_kv_heads=2,
                         head_dim=16, q_dtype="bf16", kv_dtype="fp8", fp8_mode="codes")
    for b, c in enumerate(wl.context_lens):
        for i in range(oracle.pages_for(int(c)) - 1):
            blk = wl.block_tables[b, i]
            codes = wl.k_cache[blk]
            if i * 16 + 16 < c:
                assert not ((codes & 0x7F) == 0x7F).any()


def test_validators_reject_bad_inputs():
    with pytest.raises(ValueError):
        W.validate_tables(np.array([[0, 99]]), np.array([20]), 10)
    with pytest.raises(ValueError):
        W.validate_tables(np.array([[0]]), np.array([20]), 10)
    with pytest.raises(ValueError):
        W.validate_slots(np.array([3, 3]), 10)
    with pytest.raises(ValueError):
        W.validate_copy_pairs(np.array([[1, 2], [2, 3]]), 10)
    with pytest.raises(ValueError):
        W.validate_copy_pairs(np.array([[1, 2], [4, 2]]), 10)


def test_seeded_generation_is_reproducible():
    a = W.make_workload(name="a", seed=17, context_lens=[5, 40], num_q_heads=4, num_kv_heads=2,
                        head_dim=16, q_dtype="bf16", kv_dtype="bf16")
    b = W.make_workload(name="a", seed=17, context_lens=[5, 40], num_q_heads=4, num_kv_heads=2,
                        head_dim=16, q_dtype="bf16", kv_dtype="bf16")
    for f in ("q", "k_cache", "v_cache", "block_tables", "slot_mapping", "new_k"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
