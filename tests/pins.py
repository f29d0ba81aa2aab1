"""Checks that pin the CPU oracle to things other than itself.

Each ``check_*`` raises AssertionError when the oracle disagrees with what
the pages or the mathematics fix: library routines (torch's float64 SDPA,
torch's bf16/float8_e4m3fn casts), brute force on tiny inputs, closed
forms, invariants and special cases.  The oracle is always called through
its submodules at call time, so the mutation tests can plant a mistake in
one oracle function and show that some check here catches it.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import cache_ops as co
from oracle import formats as fm
from oracle import paged_attention as pa

BLOCK = 16


# ---------------------------------------------------------------------------
# helpers that build inputs independently of the oracle's gather

def truth_sequences(rng, hkv, d, ctxs, sigma=1.0):
    """Contiguous float32 K/V per sequence, [Hkv, ctx, D] (the unpaged truth)."""
    ks = [(rng.standard_normal((hkv, c, d)) * sigma).astype(np.float32) for c in ctxs]
    vs = [(rng.standard_normal((hkv, c, d)) * sigma).astype(np.float32) for c in ctxs]
    return ks, vs


def page_out(rng, ks, vs, spare_blocks=3):
    """Place each sequence's tokens one by one into blocks taken from a shuffled pool.

    Returns pool caches (NaN where nothing was placed) and block tables
    (padding entries point at a never-used block).
    """
    hkv, d = ks[0].shape[0], ks[0].shape[2]
    need = sum(-(-k.shape[1] // BLOCK) for k in ks)
    nb = need + spare_blocks
    order = list(rng.permutation(nb))
    kc = np.full((nb, hkv, BLOCK, d), np.nan, dtype=np.float32)
    vc = np.full((nb, hkv, BLOCK, d), np.nan, dtype=np.float32)
    width = max(-(-k.shape[1] // BLOCK) for k in ks)
    tables = []
    for k, v in zip(ks, vs):
        table = []
        for t in range(k.shape[1]):
            if t % BLOCK == 0:
                table.append(order.pop(0))
            blk = table[-1]
            kc[blk, :, t % BLOCK, :] = k[:, t, :]
            vc[blk, :, t % BLOCK, :] = v[:, t, :]
        tables.append(table)
    pad = order[0]
    bt = np.full((len(ks), width), pad, dtype=np.int32)
    for i, t in enumerate(tables):
        bt[i, :len(t)] = t
    return kc, vc, bt


def sdpa_f64(q, k, v, scale):
    """torch float64 SDPA for one query row per head; KV heads repeated for GQA."""
    hq, d = q.shape
    hkv = k.shape[0]
    g = hq // hkv
    qt = torch.from_numpy(np.asarray(q, np.float64)).reshape(1, hq, 1, d)
    kt = torch.from_numpy(np.asarray(k, np.float64)).repeat_interleave(g, dim=0).unsqueeze(0)
    vt = torch.from_numpy(np.asarray(v, np.float64)).repeat_interleave(g, dim=0).unsqueeze(0)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return out.reshape(hq, d).numpy()


# ---------------------------------------------------------------------------
# attention

SDPA_CASES = [
    # (seed, Hq, Hkv, D, context lengths)
    (11, 4, 4, 16, [1, 15, 16, 17]),
    (12, 8, 2, 32, [33, 5, 48]),
    (13, 8, 1, 64, [40]),
    (14, 16, 2, 128, [31, 64, 2]),
    (15, 12, 4, 16, [100, 7]),
]


def check_decode_vs_sdpa(cases=SDPA_CASES, tol=1e-12):
    for seed, hq, hkv, d, ctxs in cases:
        rng = np.random.default_rng(seed)
        ks, vs = truth_sequences(rng, hkv, d, ctxs)
        q = rng.standard_normal((len(ctxs), hq, d)).astype(np.float32)
        kc, vc, bt = page_out(rng, ks, vs)
        scale = d ** -0.5
        got = pa.decode_ref(q, kc, vc, bt, np.array(ctxs), scale, "f32", "f32")
        for b in range(len(ctxs)):
            want = sdpa_f64(q[b], ks[b], vs[b], scale)
            err = np.abs(got[b] - want).max()
            assert err < tol, f"case seed={seed} seq={b}: |oracle - sdpa| = {err}"


def check_decode_vs_python_bruteforce():
    """Pure-Python loops (math.exp) on a tiny GQA case, against the paged oracle."""
    rng = np.random.default_rng(21)
    hq, hkv, d, ctxs = 4, 2, 4, [3, 17, 20]
    ks, vs = truth_sequences(rng, hkv, d, ctxs)
    q = rng.standard_normal((len(ctxs), hq, d)).astype(np.float32)
    kc, vc, bt = page_out(rng, ks, vs)
    scale = 0.37
    got = pa.decode_ref(q, kc, vc, bt, np.array(ctxs), scale, "f32", "f32")
    for b, ctx in enumerate(ctxs):
        for h in range(hq):
            g = h // (hq // hkv)
            logits = [scale * sum(float(q[b, h, i]) * float(ks[b][g, t, i]) for i in range(d))
                      for t in range(ctx)]
            top = max(logits)
            w = [math.exp(s - top) for s in logits]
            for i in range(d):
                want = sum(w[t] * float(vs[b][g, t, i]) for t in range(ctx)) / sum(w)
                assert abs(got[b, h, i] - want) < 1e-12, (b, h, i, got[b, h, i], want)


def check_permutation_invariance():
    """Relabelling physical blocks (and moving their contents) changes no output bit."""
    rng = np.random.default_rng(31)
    hq, hkv, d, ctxs = 8, 4, 32, [17, 64, 3, 40]
    ks, vs = truth_sequences(rng, hkv, d, ctxs)
    q = rng.standard_normal((len(ctxs), hq, d)).astype(np.float32)
    kc, vc, bt = page_out(rng, ks, vs)
    ctx = np.array(ctxs)
    base = pa.decode_ref(q, kc, vc, bt, ctx, 0.2, "f32", "f32")
    for trial in range(3):
        perm = rng.permutation(kc.shape[0])
        kc2 = np.empty_like(kc)
        vc2 = np.empty_like(vc)
        kc2[perm] = kc
        vc2[perm] = vc
        bt2 = perm[bt].astype(np.int32)
        got = pa.decode_ref(q, kc2, vc2, bt2, ctx, 0.2, "f32", "f32")
        assert np.array_equal(got.view(np.uint64), base.view(np.uint64)), f"trial {trial}"


def check_shared_prefix_equivalence():
    """Samples that share prefix blocks decode bit-identically to ones holding private copies."""
    rng = np.random.default_rng(41)
    hq, hkv, d = 4, 2, 16
    prefix, n_samples = 37, 3
    pk, pv = truth_sequences(rng, hkv, d, [prefix])
    suffixes = [5, 12, 30]
    ks, vs = [], []
    for s in suffixes:
        sk, sv = truth_sequences(rng, hkv, d, [s])
        ks.append(np.concatenate([pk[0], sk[0]], axis=1))
        vs.append(np.concatenate([pv[0], sv[0]], axis=1))
    q = rng.standard_normal((n_samples, hq, d)).astype(np.float32)
    ctx = np.array([prefix + s for s in suffixes])
    # duplicated layout: every sample owns all its blocks
    kc, vc, bt = page_out(rng, ks, vs)
    dup = pa.decode_ref(q, kc, vc, bt, ctx, 0.25, "f32", "f32")
    # shared layout: full prefix blocks stored once; the partial prefix block is private
    full = prefix // BLOCK
    shared_k = np.full((64, hkv, BLOCK, d), np.nan, np.float32)
    shared_v = np.full_like(shared_k, np.nan)
    free = list(rng.permutation(64))
    pblocks = [free.pop() for _ in range(full)]
    for i, blk in enumerate(pblocks):
        shared_k[blk] = pk[0][:, i * BLOCK:(i + 1) * BLOCK, :]
        shared_v[blk] = pv[0][:, i * BLOCK:(i + 1) * BLOCK, :]
    tables = []
    for b in range(n_samples):
        table = list(pblocks)
        for t in range(full * BLOCK, ctx[b]):
            if t % BLOCK == 0:
                table.append(free.pop())
            shared_k[table[-1], :, t % BLOCK, :] = ks[b][:, t, :]
            shared_v[table[-1], :, t % BLOCK, :] = vs[b][:, t, :]
        tables.append(table)
    bt2 = np.full((n_samples, max(len(t) for t in tables)), free[0], np.int32)
    for b, t in enumerate(tables):
        bt2[b, :len(t)] = t
    shared = pa.decode_ref(q, shared_k, shared_v, bt2, ctx, 0.25, "f32", "f32")
    assert np.array_equal(shared.view(np.uint64), dup.view(np.uint64))


def check_special_cases():
    rng = np.random.default_rng(51)
    hq, hkv, d = 4, 2, 8
    # one cached token: the output is that token's value row, exactly
    ks, vs = truth_sequences(rng, hkv, d, [1])
    q = rng.standard_normal((1, hq, d)).astype(np.float32)
    kc, vc, bt = page_out(rng, ks, vs)
    out = pa.decode_ref(q, kc, vc, bt, np.array([1]), 0.3, "f32", "f32")[0]
    for h in range(hq):
        assert np.array_equal(out[h], vs[0][h // 2, 0].astype(np.float64))
    # zero query: uniform weights -> mean of V
    ks, vs = truth_sequences(rng, hkv, d, [29])
    kc, vc, bt = page_out(rng, ks, vs)
    out = pa.decode_ref(np.zeros((1, hq, d), np.float32), kc, vc, bt, np.array([29]), 0.3, "f32", "f32")[0]
    for h in range(hq):
        assert np.abs(out[h] - vs[0][h // 2].astype(np.float64).mean(axis=0)).max() < 1e-14
    # identical keys: uniform weights -> mean of V
    ks[0][:] = ks[0][:, :1, :]
    kc, vc, bt = page_out(rng, ks, vs)
    out = pa.decode_ref(q, kc, vc, bt, np.array([29]), 0.3, "f32", "f32")[0]
    for h in range(hq):
        assert np.abs(out[h] - vs[0][h // 2].astype(np.float64).mean(axis=0)).max() < 1e-14
    # one dominant logit: the output is that token's value row
    ks, vs = truth_sequences(rng, hkv, d, [40])
    j = 23
    qq = np.zeros((1, hq, d), np.float32)
    qq[0, :, 0] = 1.0
    ks[0][:, :, 0] = 0.0
    ks[0][:, j, 0] = 1000.0
    kc, vc, bt = page_out(rng, ks, vs)
    out = pa.decode_ref(qq, kc, vc, bt, np.array([40]), 1.0, "f32", "f32")[0]
    for h in range(hq):
        assert np.abs(out[h] - vs[0][h // 2, j]).max() < 1e-12


def check_lse():
    """lse = log sum exp(scaled logits), against scipy's logsumexp."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(61)
    hq, hkv, d, ctxs = 4, 1, 16, [50, 9]
    ks, vs = truth_sequences(rng, hkv, d, ctxs)
    q = rng.standard_normal((2, hq, d)).astype(np.float32)
    kc, vc, bt = page_out(rng, ks, vs)
    _, lse = pa.decode_ref(q, kc, vc, bt, np.array(ctxs), 0.5, "f32", "f32", with_lse=True)
    for b in range(2):
        for h in range(hq):
            s = 0.5 * (ks[b][0].astype(np.float64) @ q[b, h].astype(np.float64))
            assert abs(lse[b, h] - logsumexp(s)) < 1e-12


def check_partition_merge(tol=1e-12):
    """Splitting the context into partitions and merging by log-sum-exp equals no split."""
    rng = np.random.default_rng(71)
    hq, hkv, d, ctxs = 8, 2, 32, [1, 16, 17, 100, 513, 260]
    ks, vs = truth_sequences(rng, hkv, d, ctxs)
    q = rng.standard_normal((len(ctxs), hq, d)).astype(np.float32)
    kc, vc, bt = page_out(rng, ks, vs)
    ctx = np.array(ctxs)
    whole = pa.decode_ref(q, kc, vc, bt, ctx, 0.2, "f32", "f32")
    for p in (16, 32, 48, 256, 512, 1024):
        parts = pa.decode_partitioned_ref(q, kc, vc, bt, ctx, 0.2, "f32", "f32", p)
        err = np.abs(parts - whole).max()
        assert err < tol, f"partition {p}: {err}"
    # an empty partition (m = -inf, l = 0) contributes nothing
    m = np.array([0.5, -np.inf, 1.5])
    l = np.array([2.0, 0.0, 3.0])
    acc = np.array([[1.0, 2.0], [np.nan, np.nan], [3.0, 5.0]])
    want = (math.exp(-1.0) * acc[0] + acc[2]) / (math.exp(-1.0) * 2.0 + 3.0)
    assert np.abs(pa.lse_merge_ref(m, l, acc) - want).max() < 1e-15


# ---------------------------------------------------------------------------
# number formats

def check_e4m3_table_vs_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fm.e4m3_table()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def check_e4m3_known_values():
    """Values fixed by the format definition (bias 7, 3 mantissa bits, max 448)."""
    expect = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
              0x3C: 1.5, 0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0xB8: -1.0, 0xFE: -448.0}
    for code, val in expect.items():
        assert fm.e4m3_value(code) == val, (hex(code), fm.e4m3_value(code), val)
    assert math.isnan(fm.e4m3_value(0x7F)) and math.isnan(fm.e4m3_value(0xFF))
    assert math.copysign(1.0, fm.e4m3_value(0x80)) == -1.0


def _bruteforce_e4m3(x: float) -> int:
    """Nearest finite e4m3 value by exhaustive search; ties to the even code; saturate."""
    if math.isnan(x):
        return 0x7F | (0x80 if math.copysign(1.0, x) < 0 else 0)
    best, best_err = None, None
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        v = fm.e4m3_value(c)
        if (v == 0.0) and (math.copysign(1.0, v) != math.copysign(1.0, x)):
            continue
        if v != 0.0 and (v < 0) != (x < 0):
            continue
        err = abs(v - x)
        if best is None or err < best_err or (err == best_err and (c & 1) == 0 and (best & 1) == 1):
            best, best_err = c, err
    return best


def e4m3_probe_values():
    finite = sorted({fm.e4m3_value(c) for c in range(128) if c != 0x7F})
    vals = list(finite)
    vals += [(a + b) / 2 for a, b in zip(finite, finite[1:])]            # every tie
    vals += [np.nextafter(np.float32(m), np.float32(np.inf)) for m in vals[len(finite):]]
    vals += [np.nextafter(np.float32(m), np.float32(0)) for m in vals[len(finite):2 * len(finite) - 1]]
    rng = np.random.default_rng(81)
    vals += list(np.exp2(rng.uniform(-12, 9.5, 400)))
    vals += [447.9, 448.0, 460.0, 464.0, 470.0, 1e6, 2.0 ** -10, 2.0 ** -11, 1e-30]
    vals = np.array(vals, dtype=np.float32)
    return np.concatenate([vals, -vals])


def check_e4m3_encode_bruteforce():
    vals = e4m3_probe_values()
    got = fm.e4m3_encode(vals)
    for x, c in zip(vals, got):
        want = _bruteforce_e4m3(float(x))
        assert int(c) == want, (float(x), hex(int(c)), hex(want))
    assert fm.e4m3_encode(np.array([np.inf], np.float32))[0] == 0x7E
    assert fm.e4m3_encode(np.array([-np.inf], np.float32))[0] == 0xFE
    assert (fm.e4m3_encode(np.array([np.nan], np.float32))[0] & 0x7F) == 0x7F


def check_e4m3_encode_vs_torch():
    rng = np.random.default_rng(91)
    x = np.concatenate([e4m3_probe_values(),
                        (rng.standard_normal(20000) * rng.choice([1e-3, 1.0, 100.0], 20000)).astype(np.float32)])
    clamped = np.clip(x, -448.0, 448.0).astype(np.float32)
    want = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = fm.e4m3_encode(x)
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:10]


def check_e4m3_quantize_division():
    """quantize uses the IEEE binary32 quotient (torch float32 division as the library check)."""
    rng = np.random.default_rng(92)
    x = rng.standard_normal(5000).astype(np.float32)
    s = np.exp2(rng.uniform(-10, 0, 5000)).astype(np.float32)
    qt = (torch.from_numpy(x) / torch.from_numpy(s)).clamp(-448, 448)
    want = qt.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fm.e4m3_quantize(x, s), want)


def check_bf16_vs_torch():
    rng = np.random.default_rng(101)
    bits = rng.integers(0, 65536, 20000, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp != 0xFF]
    want = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(fm.bf16_to_f64(bits), want)


def check_fp8_scaled_decode():
    """Decoding an fp8 cache equals decoding the f32 cache of code value x scale (torch decode)."""
    rng = np.random.default_rng(111)
    hq, hkv, d, nb = 4, 2, 16, 12
    ctxs = [20, 33]
    codes_k = rng.integers(0, 256, (nb, hkv, BLOCK, d), dtype=np.uint32).astype(np.uint8)
    codes_v = rng.integers(0, 256, (nb, hkv, BLOCK, d), dtype=np.uint32).astype(np.uint8)
    codes_k[(codes_k & 0x7F) == 0x7F] = 0
    codes_v[(codes_v & 0x7F) == 0x7F] = 0
    ks = np.exp2(rng.uniform(-9, -5, (nb, hkv))).astype(np.float32)
    vs = np.exp2(rng.uniform(-9, -5, (nb, hkv))).astype(np.float32)
    bt = rng.permutation(nb)[:6].reshape(2, 3).astype(np.int32)
    q = rng.standard_normal((2, hq, d)).astype(np.float32)
    got = pa.decode_ref(q, codes_k, codes_v, bt, np.array(ctxs), 0.25, "f32", "fp8", ks, vs)
    tk = torch.from_numpy(codes_k).view(torch.float8_e4m3fn).to(torch.float64).numpy() * ks[:, :, None, None]
    tv = torch.from_numpy(codes_v).view(torch.float8_e4m3fn).to(torch.float64).numpy() * vs[:, :, None, None]
    for b in range(2):
        n = -(-ctxs[b] // BLOCK)
        kk = tk[bt[b, :n]].transpose(1, 0, 2, 3).reshape(hkv, -1, d)[:, :ctxs[b]]
        vv = tv[bt[b, :n]].transpose(1, 0, 2, 3).reshape(hkv, -1, d)[:, :ctxs[b]]
        want = sdpa_f64(q[b], kk, vv, 0.25)
        assert np.abs(got[b] - want).max() < 1e-12


# ---------------------------------------------------------------------------
# cache mutation references

class ContiguousKVCache:
    """A contiguous per-layer cache [layers, heads, max_seq, head_dim] that appends
    new tokens at the current length (the layout of the pages' KV cache walk-through)."""

    def __init__(self, layers, heads, head_dim, max_seq, dtype):
        self.k = np.zeros((layers, heads, max_seq, head_dim), dtype)
        self.v = np.zeros((layers, heads, max_seq, head_dim), dtype)
        self.length = 0

    def append(self, layer, new_k, new_v):
        n = new_k.shape[1]
        self.k[layer, :, self.length:self.length + n] = new_k
        self.v[layer, :, self.length:self.length + n] = new_v
        self.length += n


def check_cache_write_vs_contiguous_append():
    """Writing tokens through slot mapping gives, read back in logical order,
    the same cache as appending them to a contiguous cache."""
    rng = np.random.default_rng(121)
    hkv, d, nb = 2, 8, 10
    n_tok = 37
    table = list(rng.permutation(nb)[:3])
    pool_k = np.full((nb, hkv, BLOCK, d), np.nan, np.float32)
    pool_v = np.full_like(pool_k, np.nan)
    before_k, before_v = pool_k.copy(), pool_v.copy()
    ref = ContiguousKVCache(1, hkv, d, 48, np.float32)
    for t in range(n_tok):
        nk = rng.standard_normal((1, hkv, d)).astype(np.float32)
        nv = rng.standard_normal((1, hkv, d)).astype(np.float32)
        slot = np.array([table[t // BLOCK] * BLOCK + t % BLOCK], np.int64)
        pool_k, pool_v = co.cache_write_ref(pool_k, pool_v, nk, nv, slot, "f32", "f32")
        ref.append(0, nk.transpose(1, 0, 2), nv.transpose(1, 0, 2))
    for t in range(n_tok):
        blk, off = table[t // BLOCK], t % BLOCK
        assert np.array_equal(pool_k[blk, :, off], ref.k[0, :, t])
        assert np.array_equal(pool_v[blk, :, off], ref.v[0, :, t])
    # nothing else was touched
    touched = np.zeros(pool_k.shape[:3], bool)
    for t in range(n_tok):
        touched[table[t // BLOCK], :, t % BLOCK] = True
    assert np.isnan(pool_k[~touched]).all() and np.isnan(pool_v[~touched]).all()
    # negative slots are skipped
    k2, v2 = co.cache_write_ref(before_k, before_v, np.ones((2, hkv, d), np.float32),
                                np.ones((2, hkv, d), np.float32), np.array([-1, -5]), "f32", "f32")
    assert np.isnan(k2).all() and np.isnan(v2).all()
    # fp8: each written value is the saturating RNE code of x / scale (torch cast as the check)
    codes = np.zeros((nb, hkv, BLOCK, d), np.uint8)
    ksc = np.exp2(rng.uniform(-9, -6, (nb, hkv))).astype(np.float32)
    vsc = np.exp2(rng.uniform(-9, -6, (nb, hkv))).astype(np.float32)
    nk = rng.standard_normal((3, hkv, d)).astype(np.float32)
    nv = rng.standard_normal((3, hkv, d)).astype(np.float32)
    slots = np.array([5, 3 * BLOCK + 15, 7 * BLOCK])
    kq, vq = co.cache_write_ref(codes, codes, nk, nv, slots, "f32", "fp8", ksc, vsc)
    for t, s in enumerate(slots):
        blk, off = s // BLOCK, s % BLOCK
        want = (torch.from_numpy(nk[t]) / torch.from_numpy(ksc[blk])[:, None]).clamp(-448, 448)
        assert np.array_equal(kq[blk, :, off], want.to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def check_copy_blocks():
    rng = np.random.default_rng(131)
    nb, hkv, d = 12, 2, 8
    kc = rng.standard_normal((nb, hkv, BLOCK, d)).astype(np.float32)
    vc = rng.standard_normal((nb, hkv, BLOCK, d)).astype(np.float32)
    ks = rng.random((nb, hkv)).astype(np.float32)
    vs = rng.random((nb, hkv)).astype(np.float32)
    pairs = np.array([[1, 7], [4, 2], [1, 9]], np.int32)
    k2, v2, ks2, vs2 = co.copy_blocks_ref(kc, vc, pairs, ks, vs)
    for blk in range(nb):
        src = {7: 1, 2: 4, 9: 1}.get(blk, blk)
        assert np.array_equal(k2[blk], kc[src]) and np.array_equal(v2[blk], vc[src])
        assert np.array_equal(ks2[blk], ks[src]) and np.array_equal(vs2[blk], vs[src])


# ---------------------------------------------------------------------------
# several new query tokens per sequence (chunked prefill, draft verification)

def pack_queries(rng, hq, d, q_lens):
    q = rng.standard_normal((int(sum(q_lens)), hq, d)).astype(np.float32)
    q_start = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    return q, q_start


def check_multi_query_full_prefill_vs_sdpa_causal(tol=1e-12):
    """q_len = ctx (a whole prompt): torch float64 SDPA with is_causal=True."""
    for seed, hq, hkv, d, ctxs in [(141, 4, 4, 16, [1, 16, 17]), (142, 8, 2, 32, [33, 5]),
                                   (143, 16, 2, 64, [40])]:
        rng = np.random.default_rng(seed)
        ks, vs = truth_sequences(rng, hkv, d, ctxs)
        q, q_start = pack_queries(rng, hq, d, ctxs)
        kc, vc, bt = page_out(rng, ks, vs)
        scale = d ** -0.5
        got = pa.multi_query_ref(q, q_start, kc, vc, bt, np.array(ctxs), scale, "f32", "f32")
        g = hq // hkv
        for b, ctx in enumerate(ctxs):
            qt = torch.from_numpy(q[q_start[b]:q_start[b + 1]].astype(np.float64)).permute(1, 0, 2)[None]
            kt = torch.from_numpy(ks[b].astype(np.float64)).repeat_interleave(g, dim=0)[None]
            vt = torch.from_numpy(vs[b].astype(np.float64)).repeat_interleave(g, dim=0)[None]
            want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
            want = want[0].permute(1, 0, 2).numpy()
            err = np.abs(got[q_start[b]:q_start[b + 1]] - want).max()
            assert err < tol, f"seed={seed} seq={b}: |oracle - sdpa causal| = {err}"


def check_multi_query_vs_python_bruteforce():
    """q_len < ctx: pure-Python loops; token i of the chunk sees positions <= ctx - q_len + i."""
    rng = np.random.default_rng(144)
    hq, hkv, d, ctxs, q_lens = 4, 2, 4, [20, 9, 33], [3, 1, 5]
    ks, vs = truth_sequences(rng, hkv, d, ctxs)
    q, q_start = pack_queries(rng, hq, d, q_lens)
    kc, vc, bt = page_out(rng, ks, vs)
    scale = 0.41
    got = pa.multi_query_ref(q, q_start, kc, vc, bt, np.array(ctxs), scale, "f32", "f32")
    for b, (ctx, ql) in enumerate(zip(ctxs, q_lens)):
        for i in range(ql):
            row = int(q_start[b]) + i
            visible = ctx - ql + i + 1
            for h in range(hq):
                g = h // (hq // hkv)
                logits = [scale * sum(float(q[row, h, j]) * float(ks[b][g, t, j]) for j in range(d))
                          for t in range(visible)]
                top = max(logits)
                w = [math.exp(s - top) for s in logits]
                for j in range(d):
                    want = sum(w[t] * float(vs[b][g, t, j]) for t in range(visible)) / sum(w)
                    assert abs(got[row, h, j] - want) < 1e-12, (b, i, h, j, got[row, h, j], want)


def check_multi_query_chunking_and_decode():
    """Cutting the new tokens into two chunks (the first chunk seeing a shorter
    context) changes nothing, and each token equals a one-token decode at its
    position: chunked prefill and token-by-token decode agree."""
    rng = np.random.default_rng(145)
    hq, hkv, d, ctxs, q_lens = 8, 2, 16, [50, 37], [7, 37]
    ks, vs = truth_sequences(rng, hkv, d, ctxs)
    q, q_start = pack_queries(rng, hq, d, q_lens)
    kc, vc, bt = page_out(rng, ks, vs)
    scale = d ** -0.5
    whole = pa.multi_query_ref(q, q_start, kc, vc, bt, np.array(ctxs), scale, "f32", "f32")
    for b, (ctx, ql) in enumerate(zip(ctxs, q_lens)):
        rows = q[q_start[b]:q_start[b + 1]]
        cut = ql // 2
        first = pa.multi_query_ref(rows[:cut], np.array([0, cut]), kc, vc, bt[b:b + 1],
                                   np.array([ctx - (ql - cut)]), scale, "f32", "f32")
        second = pa.multi_query_ref(rows[cut:], np.array([0, ql - cut]), kc, vc, bt[b:b + 1],
                                    np.array([ctx]), scale, "f32", "f32")
        both = np.concatenate([first, second])
        assert np.array_equal(both, whole[q_start[b]:q_start[b + 1]]), f"chunking changed sequence {b}"
        for i in range(ql):
            pos = ctx - ql + i
            one = pa.decode_ref(rows[i:i + 1], kc, vc, bt[b:b + 1], np.array([pos + 1]), scale, "f32", "f32")
            assert np.array_equal(one[0], whole[q_start[b] + i]), f"token {i} of sequence {b} != decode"


# ---------------------------------------------------------------------------
# int4 KV

def check_int4_encode_bruteforce():
    """Nearest of the 16 levels -8..7, ties to the even level, clamped; every tie point tried."""
    xs = np.concatenate([np.arange(-10.0, 10.01, 0.25), np.random.default_rng(151).uniform(-12, 12, 500)])
    codes = fm.int4_encode(xs.astype(np.float32))
    for x, c in zip(xs.astype(np.float32), codes):
        levels = np.arange(-8, 8)
        d = np.abs(levels - float(x))
        best = levels[d == d.min()]
        want = best[0] if len(best) == 1 else [v for v in best if v % 2 == 0][0]
        assert int(c) - 8 == want, (float(x), int(c) - 8, want)


def check_int4_nonfinite():
    """NaN has no int4 code: it is stored as -8, the value the clamp gives it
    under IEEE-754 maxNum/minNum (which return the operand that is not NaN);
    infinities saturate.  torch.fmax/fmin implement those two operations."""
    xs = np.array([np.nan, -np.nan, np.inf, -np.inf, 7.5, 8.5, -8.5, -9.0, 1e30, -1e30], np.float32)
    t = torch.from_numpy(xs.astype(np.float64))
    want = (torch.fmin(torch.fmax(torch.round(t), torch.tensor(-8.0)), torch.tensor(7.0)) + 8).to(torch.uint8).numpy()
    assert np.array_equal(fm.int4_encode(xs), want), (fm.int4_encode(xs), want)
    assert int(fm.int4_encode(np.array([np.nan], np.float32))[0]) == 0


def check_int4_layout():
    """Element 2i is the low nibble of byte i; stored code = value + 8."""
    assert list(fm.int4_to_f64(np.array([0x1F, 0x80], np.uint8))) == [7.0, -7.0, -8.0, 0.0]
    codes = np.random.default_rng(152).integers(0, 16, size=(3, 64)).astype(np.uint8)
    assert np.array_equal(fm.int4_unpack(fm.int4_pack(codes)), codes)


def check_int4_decode_vs_sdpa(tol=1e-12):
    """Decode over an int4 pool equals SDPA on values decoded independently
    (torch bit operations on the packed bytes, times the scales)."""
    rng = np.random.default_rng(153)
    hq, hkv, d, ctxs = 8, 2, 16, [5, 16, 37]
    nb = sum(-(-c // BLOCK) for c in ctxs) + 2
    kc = rng.integers(0, 256, size=(nb, hkv, BLOCK, d // 2)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(nb, hkv, BLOCK, d // 2)).astype(np.uint8)
    ks = rng.uniform(0.05, 0.5, size=(nb, hkv)).astype(np.float32)
    vs = rng.uniform(0.05, 0.5, size=(nb, hkv)).astype(np.float32)
    perm = rng.permutation(nb)
    bt = np.zeros((len(ctxs), max(-(-c // BLOCK) for c in ctxs)), np.int32)
    k = 0
    for b, c in enumerate(ctxs):
        n = -(-c // BLOCK)
        bt[b, :n] = perm[k:k + n]
        k += n
    q = rng.standard_normal((len(ctxs), hq, d)).astype(np.float32)
    got = pa.decode_ref(q, kc, vc, bt, np.array(ctxs), d ** -0.5, "f32", "int4", ks, vs)

    def torch_values(cache, scales, table, ctx):
        t = torch.from_numpy(cache[table[:-(-ctx // BLOCK)]].astype(np.int64))
        lo, hi = (t & 15) - 8, (t >> 4) - 8
        vals = torch.stack([lo, hi], dim=-1).reshape(t.shape[:-1] + (d,)).double()
        vals = vals * torch.from_numpy(scales[table[:-(-ctx // BLOCK)]].astype(np.float64))[:, :, None, None]
        return vals.permute(1, 0, 2, 3).reshape(hkv, -1, d)[:, :ctx].numpy()

    for b, c in enumerate(ctxs):
        want = sdpa_f64(q[b], torch_values(kc, ks, bt[b], c), torch_values(vc, vs, bt[b], c), d ** -0.5)
        assert np.abs(got[b] - want).max() < tol


ALL_CHECKS = [
    check_decode_vs_sdpa, check_decode_vs_python_bruteforce, check_permutation_invariance,
    check_shared_prefix_equivalence, check_special_cases, check_lse, check_partition_merge,
    check_e4m3_table_vs_torch, check_e4m3_known_values, check_e4m3_encode_bruteforce,
    check_e4m3_encode_vs_torch, check_e4m3_quantize_division, check_bf16_vs_torch,
    check_fp8_scaled_decode, check_cache_write_vs_contiguous_append, check_copy_blocks,
    check_multi_query_full_prefill_vs_sdpa_causal, check_multi_query_vs_python_bruteforce,
    check_multi_query_chunking_and_decode, check_int4_encode_bruteforce, check_int4_nonfinite, check_int4_layout,
    check_int4_decode_vs_sdpa,
]
