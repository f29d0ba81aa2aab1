"""The host planner (pa_plan_attention, through the C ABI; no GPU needed):
coverage of every query column's causal run, record routing, XCD-aware item
order, and the plan executed on the CPU with the oracle's float64 primitives
against the oracle's direct result."""
import ctypes
import math

import numpy as np
import pytest

import oracle
import pa_workloads as W
from plan_util import check_coverage, run_plan_cpu, unpack_plan

pa = pytest.importorskip("paged_kv_cache_272_amd")


def _q_start(q_lens):
    return np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)


def _tables(ctxs, rng, pool=None):
    """Block tables with distinct random physical blocks per sequence."""
    need = sum(-(-c // 16) for c in ctxs)
    ids = rng.permutation(pool or need + 7)
    mb = max(1, max(-(-c // 16) for c in ctxs))
    bt = np.full((len(ctxs), mb), ids[-1], dtype=np.int32)
    k = 0
    for b, c in enumerate(ctxs):
        n = -(-c // 16)
        bt[b, :n] = ids[k:k + n]
        k += n
    return bt


@pytest.mark.parametrize("target", [0, 1, 7, 64, 5000])
def test_decode_plan_covers_every_column(target):
    rng = np.random.default_rng(3)
    ctxs = [1, 15, 16, 17, 300, 513, 4096, 2, 1000]
    bt = _tables(ctxs, rng)
    plan, info = pa.pa_plan_attention(np.array(ctxs), 32, 8, 128, target_slices=target)
    check_coverage(plan, info, np.arange(len(ctxs) + 1), ctxs, bt, 4)
    check_slices(plan, info)
    assert info.num_shared_groups == 0
    if target:
        assert info.num_wgs == min(target, info.block_reads)


@pytest.mark.parametrize("hq,hkv", [(32, 8), (64, 8), (8, 8), (16, 1)])
def test_multi_query_plan_covers_causal_runs(hq, hkv):
    rng = np.random.default_rng(4)
    ctxs = [40, 7, 100, 16, 33, 200, 1]
    q_lens = [5, 7, 0, 16, 1, 37, 1]
    bt = _tables(ctxs, rng)
    for target in (0, 3, 40):
        plan, info = pa.pa_plan_attention(np.array(ctxs), hq, hkv, 128, q_start=_q_start(q_lens),
                                          target_slices=target)
        check_coverage(plan, info, _q_start(q_lens), ctxs, bt, hq // hkv)
        assert info.num_q_tokens == sum(q_lens)


def test_shared_prefix_plan_reads_prefix_once():
    wl = W.make_shared_prefix_workload(name="share", seed=5, num_prompts=3, samples_per_prompt=4,
                                       prefix_tokens=64, suffix_max=40, num_q_heads=32, num_kv_heads=8,
                                       head_dim=128, with_values=False)
    ctx = wl.context_lens
    plan, info = pa.pa_plan_attention(ctx, 32, 8, 128, block_tables=wl.block_tables, share_prefix=True)
    check_coverage(plan, info, np.arange(len(ctx) + 1), ctx, wl.block_tables, 4)
    # the copy-on-write of the last prefix block leaves 3 shared blocks per prompt
    assert info.num_shared_groups == 3
    plain_plan, plain = pa.pa_plan_attention(ctx, 32, 8, 128)
    per_seq = sum(-(-int(c) // 16) for c in ctx)
    assert plain.block_reads == per_seq
    # each prompt's 3 shared blocks are read by 1 item (16 columns = 4 samples x 4 heads) instead of 4
    assert info.block_reads == per_seq - 3 * 3 * (4 - 1)


def check_slices(plan, info):
    """Workgroup x runs items wg_start[x] .. wg_start[x+1]-1 and the wide groups
    own the items after those; every item belongs to exactly one workgroup or
    wide group, the slices' block counts differ by at most one, and a wide
    group's items share sequence and first block, inside the group's run."""
    p = unpack_plan(plan, info)
    ws, it, wide = p["wg_start"], p["items"], p["wide"]
    if info.num_items == 0:
        assert info.num_wgs == 0 and info.num_wide_groups == 0
        return
    n_sliced = int(ws[-1]) if info.num_wgs else 0
    reads = 0
    if info.num_wgs:
        assert ws[0] == 0 and np.all(np.diff(ws) >= 1)
        loads = [int((it["blk_hi"][ws[x]:ws[x + 1]] - it["blk_lo"][ws[x]:ws[x + 1]]).sum())
                 for x in range(info.num_wgs)]
        assert max(loads) - min(loads) <= 1
        reads += sum(loads)
    nxt = n_sliced
    for item0, n, lo, hi in sorted(wide.tolist()):
        assert item0 == nxt and 1 <= n <= 8 and lo < hi
        sl = slice(item0, item0 + n)
        assert np.all(it["seq"][sl] == it["seq"][item0]) and np.all(it["blk_lo"][sl] == lo)
        assert np.all(it["blk_hi"][sl] <= hi) and it["blk_hi"][sl].max() == hi and np.all(it["ncols"][sl] <= 32)
        reads += int(hi - lo)
        nxt += n
    assert nxt == info.num_items and reads == info.block_reads
    check_wide_order(wide, info)


def check_wide_order(wide, info):
    """The wide groups run longest first within each chunk of gcd(groups,
    per_xcd) groups, where per_xcd = ceil(groups * KV heads / 8) workgroups go
    to one XCD, and the chunks hold the groups they held in item order: every
    group keeps the XCD it would have had unsorted."""
    ng = len(wide)
    if ng < 2:
        return
    per_xcd = -(-ng * info.num_kv_heads // 8)
    chunk = math.gcd(ng, per_xcd)
    length = wide[:, 3] - wide[:, 2]
    for c0 in range(0, ng, chunk):
        part = wide[c0:c0 + chunk]
        assert np.all(np.diff(length[c0:c0 + chunk]) <= 0), "not longest first within a chunk"
        in_order = np.sort(wide[:, 0])[c0:c0 + chunk]
        assert np.array_equal(np.sort(part[:, 0]), in_order), "a group left its chunk"


def test_default_slices_fill_the_device():
    """About 2048 waves: 256 workgroups of 8 waves for 8 KV heads, 2048 of one wave for one."""
    ctxs = np.full(64, 4096)
    for hkv, want in ((8, 256), (1, 2048), (16, 128), (4, 512)):
        plan, info = pa.pa_plan_attention(ctxs, hkv * 4 if hkv < 16 else 16, hkv, 128)
        assert info.num_wgs == want, (hkv, info.num_wgs)
        check_slices(plan, info)
    plan, info = pa.pa_plan_attention(np.array([5, 20]), 32, 8, 128)   # 3 blocks: 3 slices
    assert info.num_wgs == 3


def test_sibling_tiles_take_turns():
    """16 samples x 4 heads = 64 columns: two items of 32 columns read each piece
    of the shared prefix one after the other (adjacent items); 8 samples x 4
    heads fit one item, so each prefix block is read once."""
    wl = W.make_shared_prefix_workload(name="share16", seed=6, num_prompts=4, samples_per_prompt=16,
                                       prefix_tokens=160, suffix_max=64, num_q_heads=32, num_kv_heads=8,
                                       head_dim=128, with_values=False)
    plan, info = pa.pa_plan_attention(wl.context_lens, 32, 8, 128, block_tables=wl.block_tables,
                                      share_prefix=True, target_slices=64)
    check_coverage(plan, info, np.arange(wl.num_seqs + 1), wl.context_lens, wl.block_tables, 4)
    check_slices(plan, info)
    it = unpack_plan(plan, info)["items"]
    pairs = sum(1 for k in range(info.num_items - 1)
                if (it["seq"][k], it["blk_lo"][k]) == (it["seq"][k + 1], it["blk_lo"][k + 1])
                and it["col0"][k] != it["col0"][k + 1])
    assert pairs >= 3, pairs       # a slice boundary may cut one of the 4 pairs
    wl8 = W.make_shared_prefix_workload(name="share8", seed=6, num_prompts=4, samples_per_prompt=8,
                                        prefix_tokens=160, suffix_max=64, num_q_heads=32, num_kv_heads=8,
                                        head_dim=128, with_values=False)
    plan, info = pa.pa_plan_attention(wl8.context_lens, 32, 8, 128, block_tables=wl8.block_tables_shared,
                                      share_prefix=True)
    shared_blocks = 4 * 10
    per_seq = sum(-(-int(c) // 16) for c in wl8.context_lens)
    assert info.max_item_columns == 32
    assert info.block_reads == per_seq - shared_blocks * (8 - 1)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_plan_executed_on_cpu_matches_oracle_multi_query(kv):
    wl = W.make_multi_query_workload(name="mq", seed=7, context_lens=[40, 7, 70, 16, 33], q_lens=[5, 7, 0, 16, 2],
                                     num_q_heads=8, num_kv_heads=2, head_dim=64, kv_dtype=kv)
    if kv == "fp8":
        wl.k_cache = oracle.quantize_pool_ref(wl.k_values, wl.k_scale)
        wl.v_cache = oracle.quantize_pool_ref(wl.v_values, wl.v_scale)
    k, v = oracle.cache_write_ref(wl.k_cache, wl.v_cache, wl.new_k, wl.new_v, wl.slot_mapping, "bf16", kv,
                                  wl.k_scale, wl.v_scale)
    want = oracle.multi_query_ref(wl.q, wl.q_start, k, v, wl.block_tables, wl.context_lens, wl.scale, "bf16", kv,
                                  wl.k_scale, wl.v_scale)
    for target in (0, 2, 9):
        plan, info = pa.pa_plan_attention(wl.context_lens, 8, 2, 64, q_start=wl.q_start, target_slices=target)
        got = run_plan_cpu(plan, info, wl.q, k, v, wl.block_tables, wl.context_lens, wl.scale, "bf16", kv,
                           wl.k_scale, wl.v_scale)
        assert np.abs(got - want).max() < 1e-12


def test_shared_prefix_plan_executed_on_cpu_matches_oracle_decode():
    wl = W.make_shared_prefix_workload(name="share-cpu", seed=8, num_prompts=2, samples_per_prompt=3,
                                       prefix_tokens=48, suffix_max=30, num_q_heads=8, num_kv_heads=2,
                                       head_dim=64)
    k, v = oracle.cache_write_ref(wl.k_cache, wl.v_cache, wl.new_k, wl.new_v, wl.slot_mapping, "bf16", "bf16")
    k, v, _, _ = oracle.copy_blocks_ref(k, v, wl.copy_pairs)
    want = oracle.decode_ref(wl.q, k, v, wl.block_tables, wl.context_lens, wl.scale, "bf16", "bf16")
    plan, info = pa.pa_plan_attention(wl.context_lens, 8, 2, 64, block_tables=wl.block_tables, share_prefix=True,
                                      target_slices=5)
    assert info.num_shared_groups == 2
    got = run_plan_cpu(plan, info, wl.q, k, v, wl.block_tables, wl.context_lens, wl.scale, "bf16", "bf16")
    assert np.abs(got - want).max() < 1e-12


def test_prefill_chunk_goes_to_wide_groups():
    """4 chunks of 512 new tokens at 4096 context, group 4: 2048 columns = 64
    items of 32 columns per sequence, 16 wide groups of 4 items each; 64
    groups x 8 KV heads fill the device, so no run is cut: every item writes
    its output directly and each KV head reads each block once per group."""
    ctxs, q_lens = [4096] * 4, [512] * 4
    bt = _tables(ctxs, np.random.default_rng(11))
    plan, info = pa.pa_plan_attention(np.array(ctxs), 32, 8, 128, q_start=_q_start(q_lens))
    assert info.num_wide_groups == 64 and info.num_wgs == 0 and info.num_records == 0
    assert info.num_items == 4 * 64 and info.max_item_columns == 32
    check_slices(plan, info)
    check_coverage(plan, info, _q_start(q_lens), ctxs, bt, 4)
    # a group's run ends at its last item's horizon: chunk tokens 32g .. 32g+31 see up to 3584 + 32(g+1)
    wide = unpack_plan(plan, info)["wide"]
    assert sorted(int(h) for h in wide[:, 3]) == sorted(4 * [(3584 + 32 * (k + 1)) // 16 for k in range(16)])
    assert np.all(wide[:, 2] == 0) and info.block_reads == sum(int(h) for h in wide[:, 3])
    # 64 groups x 8 heads: one head's 64 groups per XCD, so all 64 run longest first
    assert np.all(np.diff(wide[:, 3]) <= 0) and wide[0, 3] == 256 and wide[-1, 3] == 226


@pytest.mark.parametrize("hkv,nseq", [(8, 4), (2, 4), (1, 2), (1, 3), (16, 2), (8, 3)])
def test_wide_groups_run_longest_first_within_their_xcd(hkv, nseq):
    """Causal chunks give groups of different lengths (cut into pieces when
    the groups alone would not fill the device); they are ordered longest
    first within chunks of gcd(groups, ceil(groups * KV heads / 8)), so each
    XCD starts its longest runs first and keeps the groups it had."""
    ctxs, q_lens = [4096] * nseq, [512] * nseq
    plan, info = pa.pa_plan_attention(np.array(ctxs), 4 * hkv, hkv, 128, q_start=_q_start(q_lens))
    check_slices(plan, info)                       # includes the order within chunks
    wide = unpack_plan(plan, info)["wide"]
    ng = len(wide)
    chunk = math.gcd(ng, -(-ng * hkv // 8))
    length = wide[:, 3] - wide[:, 2]
    if chunk > 1:
        unsorted_len = length[np.argsort(wide[:, 0], kind="stable")]
        moved = any(not np.array_equal(length[c:c + chunk], unsorted_len[c:c + chunk]) for c in range(0, ng, chunk))
        assert moved or np.all(length == length[0]) or all(
            np.all(np.diff(unsorted_len[c:c + chunk]) <= 0) for c in range(0, ng, chunk))


def test_short_prefill_wide_groups_are_cut_into_pieces():
    """One 128-token chunk (512 columns, 2 groups): 2 groups x 8 heads are far
    from filling the device, so each group's run is cut into pieces of at
    least 8 blocks, with partial records merged per column."""
    ctxs, q_lens = [1024], [128]
    bt = _tables(ctxs, np.random.default_rng(12))
    plan, info = pa.pa_plan_attention(np.array(ctxs), 32, 8, 128, q_start=_q_start(q_lens))
    assert info.num_wgs == 0 and info.num_wide_groups > 2 and info.num_records > 0
    wide = unpack_plan(plan, info)["wide"]
    assert np.all(wide[:, 3] - wide[:, 2] >= 8)
    check_slices(plan, info)
    check_coverage(plan, info, _q_start(q_lens), ctxs, bt, 4)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_wide_plan_executed_on_cpu_matches_oracle(kv):
    """A mix of wide groups (the 40- and 33-token chunks at group 4: 160 and
    132 columns) and sliced items (decode tokens), cut and uncut, run on the
    CPU item by item: equal to the oracle's direct result."""
    wl = W.make_multi_query_workload(name="wide", seed=13, context_lens=[300, 7, 170, 16, 90],
                                     q_lens=[40, 1, 33, 1, 2], num_q_heads=8, num_kv_heads=2, head_dim=64,
                                     kv_dtype=kv)
    if kv == "fp8":
        wl.k_cache = oracle.quantize_pool_ref(wl.k_values, wl.k_scale)
        wl.v_cache = oracle.quantize_pool_ref(wl.v_values, wl.v_scale)
    k, v = oracle.cache_write_ref(wl.k_cache, wl.v_cache, wl.new_k, wl.new_v, wl.slot_mapping, "bf16", kv,
                                  wl.k_scale, wl.v_scale)
    want = oracle.multi_query_ref(wl.q, wl.q_start, k, v, wl.block_tables, wl.context_lens, wl.scale, "bf16", kv,
                                  wl.k_scale, wl.v_scale)
    for target in (0, 3):
        plan, info = pa.pa_plan_attention(wl.context_lens, 8, 2, 64, q_start=wl.q_start, target_slices=target)
        assert info.num_wide_groups >= 2 and info.num_wgs >= 1
        check_slices(plan, info)
        check_coverage(plan, info, wl.q_start, wl.context_lens, wl.block_tables, 4)
        got = run_plan_cpu(plan, info, wl.q, k, v, wl.block_tables, wl.context_lens, wl.scale, "bf16", kv,
                           wl.k_scale, wl.v_scale)
        assert np.abs(got - want).max() < 1e-12


def test_many_samples_share_a_prefix_in_wide_groups():
    """32 samples x 4 heads = 128 columns on one shared prefix: 4 tiles, one
    wide group whose items leave records, merged with each sample's suffix."""
    wl = W.make_shared_prefix_workload(name="share32", seed=14, num_prompts=1, samples_per_prompt=32,
                                       prefix_tokens=96, suffix_max=40, num_q_heads=32, num_kv_heads=8,
                                       head_dim=128, with_values=False)
    ctx = wl.context_lens
    plan, info = pa.pa_plan_attention(ctx, 32, 8, 128, block_tables=wl.block_tables_shared, share_prefix=True)
    assert info.num_shared_groups == 1 and info.num_wide_groups >= 1 and info.num_records > 0
    check_slices(plan, info)
    check_coverage(plan, info, np.arange(len(ctx) + 1), ctx, wl.block_tables_shared, 4)


def test_planner_rejects_bad_input():
    with pytest.raises(pa.PaError) as e:                  # more new tokens than context
        pa.pa_plan_attention(np.array([3]), 8, 2, 64, q_start=np.array([0, 4]))
    assert e.value.status == -2
    with pytest.raises(pa.PaError) as e:                  # group of 32
        pa.pa_plan_attention(np.array([3]), 32, 1, 64)
    assert e.value.status == -4
    with pytest.raises(pa.PaError) as e:                  # head_dim 96
        pa.pa_plan_attention(np.array([3]), 8, 2, 96)
    assert e.value.status == -4
    with pytest.raises(pa.PaError) as e:                  # q_start not starting at 0
        pa.pa_plan_attention(np.array([3, 3]), 8, 2, 64, q_start=np.array([1, 2, 3]))
    assert e.value.status == -2
    info = pa.PlanInfo()
    ctx = np.array([5], dtype=np.int32)
    # sharing without tables, and a plan buffer that is too small
    assert pa._lib.raw_call("pa_plan_attention", None, ctx.ctypes.data, None, 1, 1, 8, 2, 64, 1, 0, None, 0,
                            ctypes.byref(info)) == -1
    buf = np.zeros(16, dtype=np.uint8)
    assert pa._lib.raw_call("pa_plan_attention", None, ctx.ctypes.data, None, 1, 1, 8, 2, 64, 0, 0,
                            buf.ctypes.data, 16, ctypes.byref(info)) == -5


def test_empty_batch_plan():
    plan, info = pa.pa_plan_attention(np.zeros(0, dtype=np.int32), 8, 2, 64)
    assert info.num_items == 0 and info.workspace_bytes == 0
