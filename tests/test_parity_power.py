"""Power of the GPU parity comparison (CPU only).

The GPU parity tests compare the library's output with the oracle's by
max abs difference against the stated bars (parity.TOL).  A comparison that
cannot fail proves nothing, so here the same comparison is applied to the
oracle's own output after planting the mistakes a paged decode kernel
plausibly makes, on the inputs the GPU tests use for exactly this purpose
(the needle recipe of pa_workloads.structured, at the shapes and lengths of
the 8B-, 70B- and long-context workloads):

* one block of the sequence left out of the gather ("drop"),
* one block gathered twice ("dup"),
* one block-table entry replaced by its neighbour ("neighbour"),
* one partition's partial result merged with twice its weight ("weight"),
* one block read with the previous block's K or V scale ("stale k/v scale"),
* an all-zero output ("zero").

Each must miss the bar by at least 5x.  Blocks are taken at the start, the
middle and the end of the longest sequence, partitions of 256 and 512
tokens.  Under the plain N(0,1)*0.5 recipe the same mistakes are invisible
at long context (one block of a 4068-token sequence moves the output by
about 2e-3); that is why the needle inputs exist.
"""
import dataclasses

import numpy as np
import pytest

import host_oracle as H
import oracle
from pa_workloads import structured as S
from parity import TOL, parity_error

MARGIN = 5.0


def slice_group(wl, g: int):
    """The workload restricted to KV head g and its query heads (their outputs
    depend on nothing else)."""
    G = wl.num_q_heads // wl.num_kv_heads
    kw = dict(q=wl.q[:, g * G:(g + 1) * G].copy(), num_q_heads=G, num_kv_heads=1,
              new_k=wl.new_k[:, g:g + 1].copy(), new_v=wl.new_v[:, g:g + 1].copy())
    for name in ("k_cache", "v_cache", "k_values", "v_values", "k_scale", "v_scale"):
        a = getattr(wl, name)
        kw[name] = None if a is None else np.ascontiguousarray(a[:, g:g + 1])
    return dataclasses.replace(wl, **kw)


def build(case: str):
    if case == "needle_8b_bf16":
        wl = S.materialize(S.needle_config(2))
    elif case == "needle_8b_int4":
        wl = S.materialize(S.needle_config(2, "int4"))
    elif case == "needle_70b_bf16":
        sw = S.needle_config(3)
        lens = sw.context_lens
        order = np.argsort(lens)
        seqs = [int(order[-1]), int(order[len(order) // 2]), int(order[len(order) // 4])]
        wl = S.materialize(sw, seqs, compact=True)
    elif case == "needle_long_fp8":
        wl = slice_group(S.materialize(S.needle_config(5), [0], compact=True), 0)
    else:
        raise ValueError(case)
    H.quantize_values(wl)
    k_ref, v_ref = H.after_write(wl)
    return wl, k_ref, v_ref


CASES = ["needle_8b_bf16", "needle_8b_int4", "needle_70b_bf16", "needle_long_fp8"]


def _table_mutant(wl, b, i, kind):
    bt, lens = wl.block_tables.copy(), wl.context_lens.copy()
    n = -(-int(lens[b]) // 16)
    row = list(bt[b, :n])
    if kind == "drop":
        del row[i]
        lens[b] -= 16
    elif kind == "dup":
        row.insert(i, row[i])
        lens[b] += 16
    elif kind == "neighbour":
        row[i] = row[i + 1]
    pad = int(wl.meta["pad_block"])
    out = np.full((bt.shape[0], max(bt.shape[1], len(row))), pad, dtype=np.int32)
    out[:, :bt.shape[1]] = bt
    out[b, :] = pad
    out[b, :len(row)] = row
    return out, lens


def _weight_mutant(wl, k_ref, v_ref, b, part_tokens, p):
    ctx = int(wl.context_lens[b])
    k = oracle.gather_kv(k_ref, wl.block_tables[b], ctx, wl.kv_dtype, wl.k_scale)
    v = oracle.gather_kv(v_ref, wl.block_tables[b], ctx, wl.kv_dtype, wl.v_scale)
    qb = oracle.to_f64(wl.q[b], wl.q_dtype)
    stats = [oracle.partition_stats(qb, k, v, wl.scale, s, min(ctx, s + part_tokens))
             for s in range(0, ctx, part_tokens)]
    m = np.stack([s[0] for s in stats], axis=1)
    l = np.stack([s[1] for s in stats], axis=1)
    acc = np.stack([s[2] for s in stats], axis=1)
    l[:, p] *= 2.0
    acc[:, p] *= 2.0
    return np.stack([oracle.lse_merge_ref(m[h], l[h], acc[h]) for h in range(m.shape[0])])


def mutants(wl, k_ref, v_ref, b):
    """(name, mutated output of sequence b) for every planted mistake."""
    ctx = int(wl.context_lens[b])
    full = ctx // 16
    picks = sorted({0, full // 2, max(0, full - 2)})
    for i in picks:
        for kind in ("drop", "dup", "neighbour"):
            if kind == "neighbour" and i + 1 >= -(-ctx // 16):
                continue
            bt, lens = _table_mutant(wl, b, i, kind)
            yield f"{kind}@{i}", H.decode(wl, k_ref, v_ref, [b], block_tables=bt, context_lens=lens)[0]
    for part in (256, 512):
        nparts = -(-ctx // part)
        if nparts < 2:
            continue
        for p in sorted({0, nparts // 2, nparts - 1}):
            yield f"weight@{part}:{p}", _weight_mutant(wl, k_ref, v_ref, b, part, p)
    if wl.kv_dtype in ("fp8", "int4"):
        blocks = wl.block_tables[b, :-(-ctx // 16)]
        for which in ("k", "v"):
            scales = wl.k_scale if which == "k" else wl.v_scale
            diff = [i for i in range(1, len(blocks)) if scales[blocks[i], 0] != scales[blocks[i - 1], 0]]
            assert diff, f"no two neighbouring blocks with different {which} scales: the mutant would be moot"
            for i in sorted({diff[0], diff[len(diff) // 2], diff[-1]}):
                stale = scales.copy()
                stale[blocks[i]] = scales[blocks[i - 1]]
                kw = {"k_scale": stale} if which == "k" else {"v_scale": stale}
                yield f"stale {which} scale@{i}", H.decode(wl, k_ref, v_ref, [b], **kw)[0]
    yield "zero", None


@pytest.mark.parametrize("case", CASES)
def test_planted_mistakes_miss_the_bar(case):
    wl, k_ref, v_ref = build(case)
    want = H.decode(wl, k_ref, v_ref)
    tol = TOL[wl.kv_dtype]
    # the correct output passes, and is not small enough for zeros to pass
    assert parity_error(want, want) == 0.0
    b = int(np.argmax(wl.context_lens))
    weakest = []
    for name, out in mutants(wl, k_ref, v_ref, b):
        err = parity_error(np.zeros_like(want[b]) if out is None else out, want[b])
        weakest.append((err / tol, name))
        assert err >= MARGIN * tol, f"{case}: planted mistake '{name}' moves the output by only {err:.3e}"
    weakest.sort()
    print(f"{case}: ctx {int(wl.context_lens[b])}, weakest mutants {weakest[:3]}")


def test_random_recipe_is_blind_at_long_context():
    """Why the needle inputs exist: under the plain recipe a dropped block of a
    4068-token sequence stays far inside the bar."""
    sw = S.make_sequence_major(name="plain", seed=12, context_lens=[4068], num_q_heads=32, num_kv_heads=8,
                               head_dim=128, kv_dtype="bf16", recipe="normal")
    wl = S.materialize(sw)
    k_ref, v_ref = H.after_write(wl)
    want = H.decode(wl, k_ref, v_ref)
    bt, lens = _table_mutant(wl, 0, 100, "drop")
    err = parity_error(H.decode(wl, k_ref, v_ref, [0], block_tables=bt, context_lens=lens)[0], want[0])
    assert err < TOL["bf16"] / 2
