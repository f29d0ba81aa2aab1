"""Pins of oracle.physical_kv_bytes (the byte count of a step that reads every
physical block once): reduces to the per-sequence count without sharing, to
one sequence's K/V for identical tables, and equals a brute-force count of
touched (block, slot) pairs."""
import numpy as np

import oracle
import pa_workloads as W


def test_no_sharing_equals_decode_bytes():
    wl = W.config2(with_values=False)
    a = oracle.physical_kv_bytes(wl.block_tables, wl.context_lens, 32, 8, 128, 2, q_rows=wl.num_seqs)
    b = oracle.decode_algorithmic_bytes(wl.context_lens, 32, 8, 128, 2, 2, 2)
    assert a == b


def test_identical_tables_count_once():
    table = np.array([[5, 9, 2]] * 4, dtype=np.int32)
    lens = np.array([40] * 4)
    got = oracle.physical_kv_bytes(table, lens, 8, 2, 64, 2, q_rows=4)
    kv = 40 * 2 * 64 * 2 * 2
    assert got == kv + 4 * 8 * 64 * 4 + 12 * 4 + 16


def test_bruteforce_touched_slots():
    wl = W.make_shared_prefix_workload(name="sz", seed=3, num_prompts=3, samples_per_prompt=5, prefix_tokens=48,
                                       suffix_max=37, num_q_heads=8, num_kv_heads=2, head_dim=64,
                                       with_values=False)
    for tables in (wl.block_tables_shared, wl.block_tables):
        touched = set()
        for b, ctx in enumerate(wl.context_lens):
            for t in range(int(ctx)):
                touched.add((int(tables[b][t // 16]), t % 16))
        pages = sum(-(-int(c) // 16) for c in wl.context_lens)
        want = len(touched) * 2 * 64 * 2 * 1 + wl.num_seqs * 8 * 64 * 4 + pages * 4 + 4 * wl.num_seqs
        want += len({blk for blk, _ in touched}) * 2 * 2 * 4
        got = oracle.physical_kv_bytes(tables, wl.context_lens, 8, 2, 64, 1, q_rows=wl.num_seqs, fp8_scales=True)
        assert got == want
