"""Worked values printed on the pages (tests/golden/pages_worked_values.json)."""
import json
import os

import numpy as np

import oracle
from pa_workloads import BlockManager

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_values.json")))


def test_kv_bytes_per_token():
    g = GOLDEN["kv_bytes_per_token_llama3_70b"]
    assert oracle.kv_bytes(g["layers"], g["kv_heads"], g["head_dim"], 1, g["bytes_per_elem"]) == g["value_bytes"]
    assert g["value_bytes"] == 320 * 1024
    g = GOLDEN["kv_bytes_per_token_per_layer"]
    assert oracle.kv_bytes(1, g["kv_heads"], g["head_dim"], 1, g["bytes_per_elem"]) == g["value_bytes"]


def test_kv_bytes_for_contexts():
    per_tok = oracle.kv_bytes(80, 8, 128, 1, 2)
    g = GOLDEN["kv_4096_tokens"]
    assert oracle.kv_bytes(80, 8, 128, g["tokens"], 2) / 2 ** 20 / 1000 == g["value"]
    g = GOLDEN["kv_4000_tokens"]
    assert oracle.kv_bytes(80, 8, 128, g["tokens"], 2) / 1024 / 1e6 == g["value"]
    g = GOLDEN["kv_128k_tokens"]
    assert oracle.kv_bytes(80, 8, 128, g["tokens"], 2) == g["value"] * 2 ** 30
    g = GOLDEN["kv_100_requests_4k"]
    assert g["requests"] * per_tok * g["tokens"] / 2 ** 20 / 1000 == g["value"]


def test_pages_per_request():
    g = GOLDEN["pages_per_request"]
    for case in g["cases"]:
        assert oracle.pages_for(case["tokens"], g["block_size"]) == case["pages"]


def test_internal_fragmentation_below_one_block():
    bound = GOLDEN["internal_fragmentation"]["max_waste_tokens_exclusive"]
    for n in range(1, 3000):
        assert 0 <= oracle.internal_waste_tokens(n) < bound


def test_gqa_reduction():
    g = GOLDEN["gqa_reduction"]
    mha = oracle.kv_bytes(80, g["q_heads"], 128, 1, 2)
    gqa = oracle.kv_bytes(80, g["kv_heads"], 128, 1, 2)
    assert mha // gqa == g["kv_reduction"] and mha % gqa == 0


def test_block_table_example_gathers_logical_order():
    """The pages' example tables ([7,3,15] and [2,9]) read back tokens in logical order."""
    tables = GOLDEN["block_table_example"]["tables"]
    rng = np.random.default_rng(7)
    nb, hkv, d = 16, 1, 4
    pool = rng.standard_normal((nb, hkv, 16, d)).astype(np.float32)
    for name, table in tables.items():
        ctx = 16 * len(table) - 3
        got = oracle.gather_kv(pool, np.array(table), ctx, "f32")
        for t in range(ctx):
            assert np.array_equal(got[0, t], pool[table[t // 16], 0, t % 16].astype(np.float64))


def test_block_manager_reuses_freed_pages():
    """Freed pages are handed out again at once (section 2.3 of the batching page)."""
    bm = BlockManager(32, list(range(32)))
    a = bm.allocate_tokens(200)
    b = bm.allocate_tokens(150)
    assert len(a) == 13 and len(b) == 10
    for blk in a:
        bm.release(blk)
    c = bm.allocate_tokens(180)
    assert set(c) <= set(a) | set(range(23, 32)) and set(c) & set(a)
