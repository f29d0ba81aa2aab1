"""Read a packed attention plan (pa_plan_attention's bytes) and run it on the
CPU with the oracle's float64 primitives: a check of the host planner's
bookkeeping (coverage, causal runs, record routing), independent of the GPU."""
from __future__ import annotations

import numpy as np

import oracle

BLOCK = 16


def _align16(n: int) -> int:
    return (n + 15) // 16 * 16


def unpack_plan(plan: np.ndarray, info) -> dict:
    """Structured views of the arrays of a packed plan."""
    items_off = 0
    cols_off = _align16(items_off + info.num_items * 32)
    rows_off = _align16(cols_off + info.num_columns * 16)
    ent_off = _align16(rows_off + info.num_merge_rows * 16)
    wg_off = _align16(ent_off + info.num_merge_entries * 4)
    wide_off = _align16(wg_off + (info.num_wgs + 1 if info.num_wgs else 0) * 4)
    raw = plan.view(np.uint8)

    def view(off, n, width):
        return raw[off:off + n * 4 * width].view(np.int32).reshape(n, width)

    items = view(items_off, info.num_items, 8)
    return {
        "items": {name: items[:, k] for k, name in enumerate(
            ("seq", "blk_lo", "blk_hi", "col0", "ncols", "kv_len", "rec0", "pad"))},
        "cols": view(cols_off, info.num_columns, 4),
        "rows": view(rows_off, info.num_merge_rows, 4),
        "entries": raw[ent_off:ent_off + info.num_merge_entries * 4].view(np.int32),
        "wg_start": raw[wg_off:wg_off + (info.num_wgs + 1 if info.num_wgs else 0) * 4].view(np.int32),
        # wide groups: (first item, items, first block, end block)
        "wide": view(wide_off, info.num_wide_groups, 4),
    }


def check_coverage(plan: np.ndarray, info, q_start, context_lens, block_tables, group: int) -> None:
    """Every (new token, head-in-group) column sees each block of [0, ceil(pos+1 / 16))
    exactly once over the items that carry it (as the same physical block), and ends
    up either written by one direct item or merged from its records."""
    p = unpack_plan(plan, info)
    it = p["items"]
    q_start = np.asarray(q_start, dtype=np.int64)
    n_tok = int(q_start[-1])
    seen = {}                                   # (q_row, j) -> list of physical blocks read
    direct = {}
    recs = {}
    for k in range(info.num_items):
        if it["ncols"][k] == 0:
            continue
        seq, lo, hi, c0, nc, rec0 = (int(it[n][k]) for n in ("seq", "blk_lo", "blk_hi", "col0", "ncols", "rec0"))
        assert 1 <= nc <= 32 and lo < hi
        for c in range(nc):
            q_row, j, horizon, _ = (int(x) for x in p["cols"][c0 + c])
            key = (q_row, j)
            for blk in range(lo, hi):
                if blk * BLOCK < horizon:
                    seen.setdefault(key, []).append(int(block_tables[seq][blk]))
            if rec0 < 0:
                assert key not in direct, f"column {key} written twice"
                direct[key] = k
            else:
                recs.setdefault(key, []).append(rec0 + c)
    merged = {}
    for q_row, j, e0, n in p["rows"]:
        merged[(int(q_row), int(j))] = sorted(int(e) for e in p["entries"][e0:e0 + n])
    for b in range(len(context_lens)):
        ctx = int(context_lens[b])
        q_len = int(q_start[b + 1] - q_start[b])
        for i in range(q_len):
            horizon = ctx - q_len + i + 1
            want = [int(block_tables[b][blk]) for blk in range(-(-horizon // BLOCK))]
            for j in range(group):
                key = (int(q_start[b]) + i, j)
                assert sorted(seen.get(key, [])) == sorted(want), f"column {key}: blocks {seen.get(key)} != {want}"
                assert (key in direct) != (key in merged), f"column {key}: direct and merged"
                if key in merged:
                    assert merged[key] == sorted(recs[key]), f"column {key}: merge entries differ from its records"
    assert len(direct) + len(merged) == n_tok * group


def run_plan_cpu(plan: np.ndarray, info, q, k_cache, v_cache, block_tables, context_lens, scale, q_dtype, kv_dtype,
                 k_scale=None, v_scale=None) -> np.ndarray:
    """Execute the plan item by item in float64 (oracle.partition_stats per
    column, oracle.lse_merge_ref for merge rows)."""
    p = unpack_plan(plan, info)
    it = p["items"]
    hq, hkv, d = info.num_q_heads, info.num_kv_heads, info.head_dim
    group = hq // hkv
    out = np.zeros((info.num_q_tokens, hq, d))
    rec_m = np.full((max(info.num_records, 1), hkv), -np.inf)
    rec_l = np.zeros((max(info.num_records, 1), hkv))
    rec_acc = np.zeros((max(info.num_records, 1), hkv, d))
    gathered = {}
    for k in range(info.num_items):
        if it["ncols"][k] == 0:
            continue
        seq, lo, hi, c0, nc, kv_len, rec0 = (int(it[n][k]) for n in
                                             ("seq", "blk_lo", "blk_hi", "col0", "ncols", "kv_len", "rec0"))
        if seq not in gathered:
            ctx = int(context_lens[seq])
            gathered[seq] = (oracle.gather_kv(k_cache, block_tables[seq], ctx, kv_dtype, k_scale),
                             oracle.gather_kv(v_cache, block_tables[seq], ctx, kv_dtype, v_scale))
        kk, vv = gathered[seq]
        for c in range(nc):
            q_row, j, horizon, _ = (int(x) for x in p["cols"][c0 + c])
            qrow = oracle.to_f64(q[q_row], q_dtype)
            t0, t1 = lo * BLOCK, min(hi * BLOCK, kv_len, horizon)
            m, l, acc = oracle.partition_stats(qrow, kk, vv, scale, t0, t1)
            for g in range(hkv):
                h = g * group + j
                if rec0 < 0:
                    out[q_row, h] = acc[h] / l[h]
                else:
                    rec_m[rec0 + c, g], rec_l[rec0 + c, g], rec_acc[rec0 + c, g] = m[h], l[h], acc[h]
    for q_row, j, e0, n in p["rows"]:
        ents = p["entries"][e0:e0 + n]
        for g in range(hkv):
            out[q_row, g * group + j] = oracle.lse_merge_ref(rec_m[ents, g], rec_l[ents, g], rec_acc[ents, g])
    return out
