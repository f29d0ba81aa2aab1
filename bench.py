#!/usr/bin/env python3
"""Paged-KV attention benchmark on one MI355X.

Default workload (decode_8b, the headline): one step = one decode step of
the Llama-3-8B-shaped layer (64 sequences, 32 query / 8 KV heads,
head_dim 128, bf16, contexts U{128..4096}): each sequence's new token is
written into its slot and the paged decode runs over the cache including
it.  By default this is one pa_decode_append call (the decode kernel writes
the new rows itself, then the log-sum-exp merge kernel runs); `--step
separate` times pa_cache_write + pa_decode instead.

Other workloads (--workload): decode_70b (256 sequences, GQA-8, lognormal
contexts), long_ctx_fp8 (8 x 131072 tokens, e4m3 KV), shared_prefix_32x8
(32 prompts x 8 samples sharing a 2000-token prefix: slot write + planned
attention reading each shared block once), verify4_8b (4 draft tokens per
sequence on the 8B batch) and chunked_prefill (4 chunks of 512 tokens
appended to 3584 cached tokens).

Inputs are seeded, synthetic and resident in HBM before timing; the K/V
pool is rotated over several copies so the 256 MB Infinity Cache cannot
hold it between steps.

Prints one JSON line: whole-step throughput (algorithmic bytes / step
time; for shared prefixes every physical block counts once), sequences/s,
fraction of the 8 TB/s HBM spec and of a measured stream-read ceiling, the
dominant kernel's roofline entry (its algorithmic bytes, or flops for the
prefill chunk, over its average duration from HIP events recorded on its
own stream during the timed steps), and the CPU oracle timed on a bounded
sample of the same workload.  After the timed region it also times steps
one by one (median and p90) and reports a 'hot' figure with one pool
reused every step, labelled as such.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

SPEC_HBM_GBPS = 8000.0
METRIC = "paged-decode KV GB/s & % of MI355X HBM peak; seqs/s (8B-shape, bs=64)"
DECODE_SOURCES = ["decode_mfma.hip", "mfma_tile.h", "pa_device.h", "pa_internal.h"]
PLANNED_SOURCES = ["attend_planned.hip", "mfma_tile.h", "pa_device.h", "pa_internal.h"]
# workload -> (dominant kernel's name, the sources it is built from)
KERNELS = {
    "decode_8b": ("decode_mfma_balanced_kernel", DECODE_SOURCES),
    "decode_70b": ("decode_mfma_balanced_kernel", DECODE_SOURCES),
    "long_ctx_fp8": ("decode_mfma_balanced_kernel", DECODE_SOURCES),
    "decode_8b_int4": ("decode_mfma_balanced_kernel", DECODE_SOURCES),
    "shared_prefix_32x8": ("attend_planned_kernel", PLANNED_SOURCES),
    "verify4_8b": ("attend_planned_kernel", PLANNED_SOURCES),
    "chunked_prefill": ("attend_wide_kernel", PLANNED_SOURCES),
    "serve_8b": ("decode_mfma_balanced_kernel", DECODE_SOURCES),
}


def kernel_source_hash(sources) -> str:
    h = hashlib.sha256()
    for name in sources:
        p = os.path.join(ROOT, "paged_kv_cache_272_amd", "csrc", name)
        if os.path.exists(p):
            h.update(name.encode())
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE) into the "
                         "HBM-traffic record the roofline entry reports, and exit")
    ap.add_argument("--workload", choices=sorted(KERNELS), default="decode_8b",
                    help="decode_8b (default) is the headline step; the others measure the other shapes and "
                         "the planned (multi-token, shared-prefix) paths")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--pools", type=int, default=3, help="K/V pool copies rotated across steps")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dist-steps", type=int, default=100,
                    help="steps timed one by one after the timed region (median, p90), and steps of the 'hot' "
                         "figure (one pool reused); 0 skips both")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--timing-every", type=int, default=8,
                    help="record HIP events around the decode kernels of one step in this many")
    ap.add_argument("--step", choices=("append", "separate"), default="append",
                    help="append: one pa_decode_append call; separate: pa_cache_write then pa_decode")
    return ap.parse_args()


def measured_stream_read(pa, torch, nbytes=4 << 30, reps=5):
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(pa.pa_probe_sink_bytes(), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        pa.pa_probe_stream_read(buf, sink)
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pa.pa_probe_stream_read(buf, sink)
        e1.record()
        e1.synchronize()
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    return best


COPY_PROBE_BYTES = 1 << 30
COPY_KERNEL = "probe_copy_kernel"


def copy_probe(pa, torch):
    """One plain copy of known size: the calibration point for the HBM byte counters."""
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    pa.pa_probe_copy(dst, src)
    torch.cuda.synchronize()


def _counter_per_dispatch(run_dir, counter):
    """{kernel-name substring: [per-dispatch value in bytes]} from a rocprofv3 counter CSV."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(path)):
            if row.get("Counter_Name") != counter:
                continue
            name = row.get("Kernel_Name", "")
            # FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch
            out.setdefault(name, []).append(float(row["Counter_Value"]) * 1024.0)
    return out


def traffic_record(workload, fetch_dir, write_dir):
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")

    def pick(table, key):
        vals = [v for name, vs in table.items() if key in name for v in vs]
        if not vals:
            raise SystemExit(f"no {key} dispatches in the counter output")
        vals.sort()
        return vals[len(vals) // 2]

    copy_read, copy_write = pick(fetch, COPY_KERNEL), pick(write, COPY_KERNEL)
    read_scale = COPY_PROBE_BYTES / copy_read
    write_scale = COPY_PROBE_BYTES / copy_write
    kernel, sources = KERNELS[workload]
    dec_read, dec_write = pick(fetch, kernel), pick(write, kernel)
    rec = {
        "workload": workload,
        "kernel": kernel,
        "kernel_source_hash": kernel_source_hash(sources),
        "fetch_bytes_per_launch_raw": dec_read, "write_bytes_per_launch_raw": dec_write,
        "copy_probe_bytes": COPY_PROBE_BYTES, "copy_probe_fetch_raw": copy_read, "copy_probe_write_raw": copy_write,
        "read_scale": read_scale, "write_scale": write_scale,
        "hbm_bytes_per_launch": round(dec_read * read_scale + dec_write * write_scale),
        "method": "rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (separate runs) over bench.py; median "
                  "per-dispatch value, each scaled by (known bytes / counter) of a 1 GiB probe copy in the "
                  "same run",
    }
    with open(traffic_file(workload), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def cpu_baseline(bench, budget_s, threads=None):
    """The oracle on a bounded sample of the same workload: whole sequences,
    cycling over the batch, until the time budget ends.  BLAS runs one thread
    per call and `threads` host threads take sequences in turn (the oracle's
    array work releases the interpreter lock)."""
    import concurrent.futures as cf
    import threading
    from threadpoolctl import threadpool_limits
    bench.cpu_prepare()
    threads = threads or max(1, min(8, os.cpu_count() or 1))
    lock = threading.Lock()
    state = {"next": 0, "done": 0, "bytes": 0}

    def worker(t_end):
        while time.perf_counter() < t_end:
            with lock:
                b = state["next"] % bench.num_seqs
                state["next"] += 1
            nb = bench.cpu_one(b)
            with lock:
                state["done"] += 1
                state["bytes"] += nb
    with threadpool_limits(limits=1):
        t_start = time.perf_counter()
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            for f in [ex.submit(worker, t_start + budget_s) for _ in range(threads)]:
                f.result()
        elapsed = time.perf_counter() - t_start
    done, nbytes = state["done"], state["bytes"]
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": round(nbytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"float64 numpy oracle ({bench.cpu_kind}) on {threads} host threads (BLAS 1 thread each), "
                  f"{done} sequences cycling over the {bench.num_seqs}-sequence batch ({nbytes / 1e6:.1f} MB "
                  f"algorithmic) in {elapsed:.1f} s; host CPU {cpu}",
        "seqs_per_s": round(done / elapsed, 3),
    }


class Bench:
    """One workload: prepared calls per pool, byte and flop counts, labels."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def _dev(torch, np, a, kind=None):
    a = np.ascontiguousarray(a)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(a).to("cuda")


def build_decode(args, pa, torch, np, W, oracle, name):
    """Decode workloads: one new token per sequence (pa_decode_append, or
    pa_cache_write + pa_decode with --step separate)."""
    def int4_8b():
        base = W.config2(with_values=False)
        return W.make_workload(name="llama3_8b_int4", seed=2, context_lens=[int(c) for c in base.context_lens],
                               num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16", kv_dtype="int4",
                               fp8_mode="codes")
    if name == "long_ctx_fp8":
        return build_long_context(args, pa, torch, np, oracle)
    wl = {"decode_8b": W.config2, "decode_70b": W.config3, "decode_8b_int4": int4_8b}[name]()
    kv = wl.kv_dtype
    q = _dev(torch, np, wl.q, "bf16")
    new_k, new_v = _dev(torch, np, wl.new_k, "bf16"), _dev(torch, np, wl.new_v, "bf16")
    bt, cl, slots = _dev(torch, np, wl.block_tables), _dev(torch, np, wl.context_lens), _dev(torch, np, wl.slot_mapping)
    k0, v0 = _dev(torch, np, wl.k_cache, kv if kv == "bf16" else None), _dev(torch, np, wl.v_cache,
                                                                            kv if kv == "bf16" else None)
    ks = None if wl.k_scale is None else _dev(torch, np, wl.k_scale)
    vs = None if wl.v_scale is None else _dev(torch, np, wl.v_scale)
    return _decode_bench(args, pa, torch, np, oracle, name, wl, q, new_k, new_v, bt, cl, slots, k0, v0, ks, vs)


def _decode_bench(args, pa, torch, np, oracle, name, wl, q, new_k, new_v, bt, cl, slots, k0, v0, ks, vs,
                  data=None, cpu_wl=None):
    kv = wl.kv_dtype
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(args.pools - 1)]
    out = torch.empty_like(q)
    ws_bytes = pa.pa_decode_workspace_size(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                           wl.max_context_len, args.partition_tokens)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    steps = []
    for kc, vc in pools:
        if args.step == "append":
            steps.append((pa.prepare_decode_append(out, q, new_k, new_v, kc, vc, bt, cl, wl.max_context_len,
                                                   wl.scale, ks, vs, partition_tokens=args.partition_tokens,
                                                   workspace=ws),))
        else:
            steps.append((pa.prepare_cache_write(new_k, new_v, kc, vc, slots, ks, vs),
                          pa.prepare_decode(out, q, kc, vc, bt, cl, wl.max_context_len, wl.scale, ks, vs,
                                            partition_tokens=args.partition_tokens, workspace=ws)))
    eb = {"fp8": 1, "int4": 0.5}.get(kv, 2)
    scaled = kv in ("fp8", "int4")
    decode_bytes = int(oracle.decode_algorithmic_bytes(wl.context_lens, wl.num_q_heads, wl.num_kv_heads,
                                                       wl.head_dim, eb, 2, 2, fp8_scales=scaled))
    write_bytes = int(wl.num_seqs * wl.num_kv_heads * wl.head_dim * (2 + eb) * 2 + wl.num_seqs * 8)
    part = pa.pa_decode_partition_tokens(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                         wl.max_context_len, args.partition_tokens)
    labels = {"decode_8b": ("llama3_8b_shape_decode_bs64", "U{128..4096}"),
              "decode_70b": ("llama3_70b_shape_decode_bs256", "lognormal median 2048 in [16, 8192]"),
              "long_ctx_fp8": ("llama3_70b_shape_fp8_decode_bs8_ctx131072", "131072 each"),
              "decode_8b_int4": ("llama3_8b_shape_int4_decode_bs64", "U{128..4096}")}[name]
    k_ref = v_ref = None

    # the CPU oracle's sample: the workload itself, or (long context) a host
    # copy of some of its sequences (cpu_wl() builds it)
    host = {}

    def cpu_prepare():
        h = wl if cpu_wl is None else cpu_wl()
        host["wl"] = h
        host["ref"] = oracle.cache_write_ref(h.k_cache, h.v_cache, h.new_k, h.new_v, h.slot_mapping, "bf16", kv,
                                             h.k_scale, h.v_scale)

    def cpu_one(b):
        h = host["wl"]
        b = b % h.num_seqs
        k_ref, v_ref = host["ref"]
        oracle.decode_ref(h.q, k_ref, v_ref, h.block_tables, h.context_lens, h.scale, "bf16", kv,
                          h.k_scale, h.v_scale, seqs=[b])
        return oracle.decode_algorithmic_bytes(h.context_lens[b:b + 1], h.num_q_heads, h.num_kv_heads,
                                               h.head_dim, eb, 2, 2, fp8_scales=scaled)

    return Bench(
        workload=labels[0], steps=steps, pools=len(pools), step_bytes=decode_bytes + write_bytes,
        kernel_bytes=decode_bytes, kernel_flops=None, num_seqs=wl.num_seqs, dtype="bf16" if kv == "bf16" else kv,
        kernel_label="decode partition kernel",
        data=data or ("synthetic (seeded N(0,1)*0.5 bf16 q/K/V, shuffled 16-token block pool)" if kv == "bf16" else
                      "synthetic (seeded bf16 q, random finite e4m3 codes with per-(block, head) scales 2^U(-8,-6))"
                      if kv == "fp8" else
                      "synthetic (seeded bf16 q, random int4 codes with per-(block, head) scales 2^U(-4,-2))"),
        config={"workload": labels[0], "batch": wl.num_seqs, "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads,
                "head_dim": wl.head_dim, "block_size": 16, "context_lens": labels[1],
                "sum_context": int(wl.context_lens.sum()), "kv_dtype": kv, "pool_blocks": wl.num_blocks,
                "pools_rotated": len(pools),
                "work_split": ("balanced slices of the (sequence, block) list" if args.partition_tokens == 0
                               else f"{part}-token partitions"),
                "step": (f"pa_decode_append: slot write of the {wl.num_seqs} new tokens fused into the decode"
                         if args.step == "append" else f"pa_cache_write({wl.num_seqs} tokens) + pa_decode")},
        cpu_prepare=cpu_prepare, cpu_one=cpu_one, cpu_kind="decode_ref")


def build_long_context(args, pa, torch, np, oracle):
    """Long-context e4m3 decode as stated: 8 x 131072 tokens, K/V N(0,1)*0.5
    drawn sequence by sequence and quantised to e4m3 on the GPU by the
    self-scaling scatter (whole blocks: one amax/448 scale per (block, KV
    head)); the newest token of each sequence is then written by the decode
    step itself."""
    from concurrent.futures import ThreadPoolExecutor
    from pa_workloads import structured as S
    swl = S.config5_sequence_major("normal")
    lay = swl.layout
    nb, hkv, d = swl.num_blocks, swl.num_kv_heads, swl.head_dim
    k0 = torch.full((nb, hkv, 16, d), 0x7F, dtype=torch.uint8, device="cuda")
    v0 = torch.full_like(k0, 0x7F)
    ks = torch.ones(nb, hkv, dtype=torch.float32, device="cuda")
    vs = torch.ones_like(ks)
    new_k = np.empty((swl.num_seqs, hkv, d), np.uint16)
    new_v = np.empty_like(new_k)
    for b, k, v in swl.iter_values():
        ctx = int(swl.context_lens[b])
        pos = np.arange(ctx, dtype=np.int64)
        slots_b = lay.block_tables[b, pos // 16].astype(np.int64) * 16 + pos % 16
        pa.pa_cache_write_autoscale(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), k0, v0, ks, vs,
                                    torch.from_numpy(slots_b).cuda())
        new_k[b], new_v[b] = S.to_bf16_bits(k[ctx - 1]), S.to_bf16_bits(v[ctx - 1])
        del k, v
    torch.cuda.synchronize()
    lay.q, lay.new_k, lay.new_v, lay.kv_dtype = swl.q, new_k, new_v, "fp8"
    q = _dev(torch, np, swl.q, "bf16")
    dnk, dnv = _dev(torch, np, new_k, "bf16"), _dev(torch, np, new_v, "bf16")
    bt, cl = _dev(torch, np, lay.block_tables), _dev(torch, np, lay.context_lens)
    slots = _dev(torch, np, lay.slot_mapping)

    def cpu_wl():
        # two sequences, quantised on the host by the oracle (input preparation, not timed)
        h = S.materialize(swl, [0, 1], compact=True)
        with ThreadPoolExecutor(S.default_workers()) as ex:
            h.k_cache, h.v_cache = ex.map(lambda t: oracle.quantize_pool_ref(*t, "fp8"),
                                          [(h.k_values, h.k_scale), (h.v_values, h.v_scale)])
        return h

    data = ("synthetic (seeded: bf16 q N(0,1)*0.5; K/V N(0,1)*0.5 drawn per sequence, quantised to e4m3 on the "
            "GPU by pa_cache_write_autoscale with one amax/448 scale per (block, KV head))")
    return _decode_bench(args, pa, torch, np, oracle, "long_ctx_fp8", lay, q, dnk, dnv, bt, cl, slots, k0, v0, ks,
                         vs, data=data, cpu_wl=cpu_wl)


def build_planned(args, pa, torch, np, W, oracle, name):
    """Planned attention workloads (host plan built once before timing; its
    build time is reported): the 32 x 8 shared-prefix decode (slot write of
    the new tokens + prefix-shared attention), draft verification of 4
    tokens per sequence on the 8B batch, and a chunked-prefill chunk."""
    share = name == "shared_prefix_32x8"
    if share:
        wl = W.config4()
        tables_host = wl.block_tables
    elif name == "verify4_8b":
        base = W.config2(with_values=False)
        wl = W.make_multi_query_workload(name=name, seed=302, context_lens=[int(c) for c in base.context_lens],
                                         q_lens=[4] * base.num_seqs, num_q_heads=32, num_kv_heads=8, head_dim=128)
        tables_host = wl.block_tables
    else:
        wl = W.make_multi_query_workload(name=name, seed=303, context_lens=[4096] * 4, q_lens=[512] * 4,
                                         num_q_heads=32, num_kv_heads=8, head_dim=128)
        tables_host = wl.block_tables
    q = _dev(torch, np, wl.q, "bf16")
    new_k, new_v = _dev(torch, np, wl.new_k, "bf16"), _dev(torch, np, wl.new_v, "bf16")
    bt, slots = _dev(torch, np, wl.block_tables), _dev(torch, np, wl.slot_mapping)
    k0, v0 = _dev(torch, np, wl.k_cache, "bf16"), _dev(torch, np, wl.v_cache, "bf16")
    copy_rate = None
    if share:
        pairs = _dev(torch, np, wl.copy_pairs.astype(np.int32))
        pa.pa_copy_blocks(k0, v0, pairs)
        # the copy-on-write call on its own: every pair's K and V block read and
        # written (repeating it rewrites the same bytes)
        copy_bytes = 2 * 2 * len(wl.copy_pairs) * wl.num_kv_heads * 16 * wl.head_dim * 2
        for _ in range(5):
            pa.pa_copy_blocks(k0, v0, pairs)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(50):
            pa.pa_copy_blocks(k0, v0, pairs)
        e1.record()
        torch.cuda.synchronize()
        copy_us = e0.elapsed_time(e1) / 50 * 1e3
        copy_rate = {"pairs": int(len(wl.copy_pairs)), "bytes_read_and_written": int(copy_bytes),
                     "us_per_call": round(copy_us, 2), "GBps": round(copy_bytes / (copy_us * 1e-6) / 1e9, 1),
                     "timing": "HIP events around 50 back-to-back calls"}
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(args.pools - 1)]
    t_plan = time.perf_counter()
    for _ in range(5):
        plan, info = pa.pa_plan_attention(wl.context_lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                          q_start=wl.q_start, block_tables=tables_host if share else None,
                                          share_prefix=share)
    plan_ms = (time.perf_counter() - t_plan) / 5 * 1e3
    dplan = pa.plan_to_device(plan)
    out = torch.empty_like(q)
    ws = torch.empty(max(info.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    steps = []
    for kc, vc in pools:
        call = pa.prepare_attend_planned(out, q, kc, vc, bt, wl.scale, dplan, info, workspace=ws)
        steps.append((pa.prepare_cache_write(new_k, new_v, kc, vc, slots), call) if share else (call,))
    q_rows = int(wl.q.shape[0])
    kernel_bytes = oracle.physical_kv_bytes(wl.block_tables, wl.context_lens, wl.num_q_heads, wl.num_kv_heads,
                                            wl.head_dim, 2, q_rows)
    logical_bytes = oracle.decode_algorithmic_bytes(wl.context_lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                                    2, 2, 2)
    write_bytes = wl.num_seqs * wl.num_kv_heads * wl.head_dim * 2 * 2 * 2 + wl.num_seqs * 8 if share else 0
    qs = wl.q_start if wl.q_start is not None else np.arange(wl.num_seqs + 1)
    horizons = np.concatenate([np.arange(int(c) - (qs[b + 1] - qs[b]) + 1, int(c) + 1)
                               for b, c in enumerate(wl.context_lens)])
    flops = 4 * wl.head_dim * wl.num_q_heads * int(horizons.sum())
    label = {"shared_prefix_32x8": "shared_prefix_32x8_decode", "verify4_8b": "llama3_8b_shape_verify4_bs64",
             "chunked_prefill": "llama3_8b_shape_prefill_chunk512_ctx4096_x4"}[name]
    k_ref = v_ref = None

    def cpu_prepare():
        nonlocal k_ref, v_ref
        k_ref, v_ref = oracle.cache_write_ref(wl.k_cache, wl.v_cache, wl.new_k, wl.new_v, wl.slot_mapping,
                                              "bf16", "bf16")
        if share:
            k_ref, v_ref, _, _ = oracle.copy_blocks_ref(k_ref, v_ref, wl.copy_pairs)

    def cpu_one(b):
        if share:
            oracle.decode_ref(wl.q, k_ref, v_ref, wl.block_tables, wl.context_lens, wl.scale, "bf16", "bf16",
                              seqs=[b])
        else:
            oracle.multi_query_ref(wl.q, wl.q_start, k_ref, v_ref, wl.block_tables, wl.context_lens, wl.scale,
                                   "bf16", "bf16", seqs=[b])
        return oracle.physical_kv_bytes(wl.block_tables[b:b + 1], wl.context_lens[b:b + 1], wl.num_q_heads,
                                        wl.num_kv_heads, wl.head_dim, 2, int(qs[b + 1] - qs[b]))

    config = {"workload": label, "batch": wl.num_seqs, "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads,
              "head_dim": wl.head_dim, "block_size": 16, "query_tokens": q_rows,
              "sum_context": int(wl.context_lens.sum()), "kv_dtype": "bf16", "pool_blocks": wl.num_blocks,
              "pools_rotated": len(pools), "plan": info.as_dict(), "plan_build_ms_host": round(plan_ms, 3),
              "logical_kv_bytes": int(logical_bytes),
              "step": ("pa_cache_write(256 tokens) + pa_attend_planned with prefix sharing (plan built on the host "
                       "before timing)" if share else
                       "pa_attend_planned over caches already holding the new tokens' K/V (plan built before timing)")}
    return Bench(
        workload=label, steps=steps, pools=len(pools), step_bytes=kernel_bytes + write_bytes,
        kernel_bytes=kernel_bytes, kernel_flops=flops, num_seqs=wl.num_seqs, dtype="bf16",
        kernel_label=("planned attention kernels (wide groups %d, sliced workgroups %d)"
                      % (info.num_wide_groups, info.num_wgs)),
        data="synthetic (seeded N(0,1)*0.5 bf16 q/K/V, shuffled 16-token block pool)", config=config,
        logical_bytes=logical_bytes, copy_blocks=copy_rate, cpu_prepare=cpu_prepare, cpu_one=cpu_one,
        cpu_kind="decode_ref" if share else "multi_query_ref", mfma_bound=name == "chunked_prefill")


WORKLOADS = {"decode_8b": build_decode, "decode_70b": build_decode, "long_ctx_fp8": build_decode,
             "decode_8b_int4": build_decode,
             "shared_prefix_32x8": build_planned, "verify4_8b": build_planned, "chunked_prefill": build_planned}


def run_serve(args, pa, torch, np, oracle):
    """Continuous batching through the library's driver (native block
    manager + pa_copy_blocks + pa_decode_append), 8B shape, up to 64 running
    sequences.  Requests arrive with a prompt of U{128..4096} tokens (its K/V
    written by pa_cache_write on admission; the prompt's attention is not
    part of this loop) and decode a lognormal number of tokens (median 256,
    clipped to [16, 2048]); finished sequences leave and waiting ones join
    between iterations; a step that does not fit preempts the newest
    sequence (freed, re-queued to be recomputed).  Timed: K iterations,
    admissions included.  Reported besides throughput: the host time per
    iteration, and KV memory use against reserving max_model_len per request."""
    from paged_kv_cache_272_amd.driver import DecodeDriver
    hq, hkv, d, slots, max_len = 32, 8, 128, 64, 4096 + 2048
    mb = max_len // 16
    rng = np.random.default_rng(501)
    num_blocks = int(slots * (2048 + 512) / 16 * 1.25)
    drv = DecodeDriver(num_blocks, hq, hkv, d, mb, max_batch=slots, free_order=rng.permutation(num_blocks))
    noise = torch.randn(4096 * hkv * d * 2, device="cuda").to(torch.bfloat16)
    kv_src = noise[:4096 * hkv * d].view(4096, hkv, d)
    q = torch.randn(slots, hq, d, device="cuda").to(torch.bfloat16)
    kn = torch.randn(slots, hkv, d, device="cuda").to(torch.bfloat16)
    vn = torch.randn(slots, hkv, d, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    state = {"next": 0, "waiting": [], "running": [], "left": {}, "ctx": {}, "admitted": 0, "finished": 0,
             "preempted": 0, "host_s": 0.0, "tokens": 0, "kv_bytes": 0, "util": [], "naive": [], "iters": 0}

    def new_request():
        n = int(rng.integers(128, 4097))
        out_len = int(np.clip(np.round(np.exp(rng.normal(np.log(256), 1.0))), 16, 2048))
        state["waiting"].append((state["next"], n, out_len))
        state["next"] += 1

    def admit():
        while len(state["running"]) < slots:
            if not state["waiting"]:
                new_request()
            seq, n, out_len = state["waiting"][0]
            try:
                drv.add_sequence(seq, kv_src[:n], kv_src[:n])
            except pa.OutOfBlocks:
                break
            state["waiting"].pop(0)
            state["running"].append(seq)
            state["left"][seq] = out_len
            state["ctx"][seq] = n
            state["admitted"] += 1

    def iteration():
        admit()
        t0 = time.perf_counter()
        while True:
            b = len(state["running"])
            try:
                drv.step(state["running"], q[:b], kn[:b], vn[:b], out[:b])
                break
            except pa.OutOfBlocks:
                victim = state["running"].pop()
                drv.finish(victim)
                state["waiting"].insert(0, (victim, state["ctx"][victim], state["left"][victim]))
                state["preempted"] += 1
        state["host_s"] += time.perf_counter() - t0
        lens = [state["ctx"][s] + 1 for s in state["running"]]
        state["tokens"] += len(lens)
        state["kv_bytes"] += int(sum(lens)) * hkv * d * 2 * 2
        for s in list(state["running"]):
            state["ctx"][s] += 1
            state["left"][s] -= 1
            if state["left"][s] <= 0:
                state["running"].remove(s)
                drv.finish(s)
                state["finished"] += 1
        state["iters"] += 1
        if state["iters"] % 8 == 1:           # memory use sampled every 8th iteration
            st = drv.bm.stats()
            used = (st["num_blocks"] - st["free_blocks"]) * 16
            state["util"].append(st["stored_tokens"] / max(used, 1))
            state["naive"].append(st["logical_tokens"] / max(len(state["running"]) * max_len, 1))

    for _ in range(args.warmup):
        iteration()
    torch.cuda.synchronize()
    for k in ("tokens", "kv_bytes", "host_s", "admitted", "finished", "preempted"):
        state[k] = 0 if k != "host_s" else 0.0
    state["util"], state["naive"] = [], []
    pa.pa_timing_read()
    pa.pa_timing_enable(args.timing_every)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        iteration()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    pa.pa_timing_enable(0)
    part_ms, merge_ms, calls = pa.pa_timing_read()
    step_s = elapsed / args.steps
    part_avg = part_ms / max(calls, 1)
    tok_s = state["tokens"] / elapsed
    result = {
        "metric": METRIC, "value": round(state["kv_bytes"] / elapsed / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random bf16 K/V and queries; lognormal output lengths)",
        "config": {"workload": "serve_8b_continuous_batching", "slots": slots, "q_heads": hq, "kv_heads": hkv,
                   "head_dim": d, "pool_blocks": num_blocks, "max_model_len": max_len,
                   "prompt_tokens": "U{128..4096}", "output_tokens": "lognormal median 256, [16, 2048]",
                   "step": "admissions (pa_cache_write of prompts) + pa_bm_step + copy-on-write + pa_decode_append"},
        "decode_tokens_per_s": round(tok_s, 1),
        "seqs_per_s": round(tok_s, 1),
        "host_ms_per_step": round(state["host_s"] / args.steps * 1e3, 4),
        "admitted": state["admitted"], "finished": state["finished"], "preempted": state["preempted"],
        "kv_memory_used_by_tokens": round(float(np.mean(state["util"])), 4),
        "kv_memory_used_by_tokens_if_reserving_max_len": round(float(np.mean(state["naive"])), 4),
        "decode_partition_kernel_ms": round(part_avg, 5),
        "decode_merge_kernel_ms": round(merge_ms / max(calls, 1), 5),
        "roofline": None, "cpu_baseline": None,
        "note": "KV GB/s counts each step's live K/V once; the decode kernel's roofline is the decode_8b leg's",
    }
    print(json.dumps(result), flush=True)


def step_distribution(torch, steps, n):
    """Median and p90 (us) of n steps, each between two HIP events on the
    launch stream, rotating the pools as the timed region does."""
    if n <= 0:
        return None, None
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        evs[i][0].record()
        for call in steps[i % len(steps)]:
            call()
        evs[i][1].record()
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return round(us[len(us) // 2], 2), round(us[min(len(us) - 1, (9 * len(us)) // 10)], 2)


def hot_step(torch, steps, n):
    """Mean step time (ms) with the first pool every step: the 'hot' figure."""
    if n <= 0:
        return None
    for _ in range(5):
        for call in steps[0]:
            call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        for call in steps[0]:
            call()
    torch.cuda.synchronize()
    return round((time.perf_counter() - t0) / n * 1e3, 5)


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def main():
    args = parse_args()
    if args.traffic_from:
        traffic_record(args.workload, *args.traffic_from)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the decode shards by sequence or KV head with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import oracle
    import paged_kv_cache_272_amd as pa
    import pa_workloads as W

    torch.cuda.set_device(0)
    if args.workload == "serve_8b":
        run_serve(args, pa, torch, np, oracle)
        return
    t_gen = time.perf_counter()
    bench = WORKLOADS[args.workload](args, pa, torch, np, W, oracle, args.workload)
    print(f"# {bench.workload}: set up in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    copy_probe(pa, torch)
    peak_meas = measured_stream_read(pa, torch)
    print(f"# measured stream read {peak_meas:.0f} GB/s", file=sys.stderr, flush=True)

    steps = bench.steps
    for i in range(args.warmup):
        for call in steps[i % len(steps)]:
            call()
    torch.cuda.synchronize()

    pa.pa_timing_read()
    pa.pa_timing_enable(args.timing_every)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for call in steps[i % len(steps)]:
            call()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    pa.pa_timing_enable(0)
    part_ms, merge_ms, calls = pa.pa_timing_read()

    step_s = (t1 - t0) / args.steps
    value = bench.step_bytes / step_s / 1e9
    dist = step_distribution(torch, steps, args.dist_steps)
    hot = hot_step(torch, steps, args.dist_steps)
    part_avg_ms = part_ms / max(calls, 1)
    merge_avg_ms = merge_ms / max(calls, 1)
    achieved = bench.kernel_bytes / (part_avg_ms * 1e-3) / 1e9

    traffic = None
    tf = traffic_file(args.workload)
    if os.path.exists(tf):
        rec = json.load(open(tf))
        if rec.get("kernel_source_hash") == kernel_source_hash(KERNELS[args.workload][1]):
            traffic = rec.get("hbm_bytes_per_launch")

    roofline = {
        "kernel": bench.kernel_label,
        "bound": "hbm", "achieved": round(achieved, 1), "peak": SPEC_HBM_GBPS, "unit": "GB/s",
        "frac": round(achieved / SPEC_HBM_GBPS, 4), "traffic": traffic,
        "algorithmic_bytes_per_launch": int(bench.kernel_bytes),
    }
    if getattr(bench, "mfma_bound", False):
        tflops = bench.kernel_flops / (part_avg_ms * 1e-3) / 1e12
        roofline.update({"bound": "mfma", "achieved": round(tflops, 2), "peak": 2500.0, "unit": "TFLOP/s",
                         "frac": round(tflops / 2500.0, 4), "algorithmic_flops_per_launch": int(bench.kernel_flops),
                         "kv_GBps": round(achieved, 1)})
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": bench.dtype,
        "data": bench.data,
        "config": bench.config,
        "seqs_per_s": round(bench.num_seqs / step_s, 1),
        "pct_of_spec_hbm": round(100 * value / SPEC_HBM_GBPS, 2),
        "measured_stream_read_GBps": round(peak_meas, 1),
        "pct_of_measured_stream_read": round(100 * value / peak_meas, 2),
        "step_algorithmic_bytes": int(bench.step_bytes),
        "step_us_median": dist[0],
        "step_us_p90": dist[1],
        "step_timing": (f"HIP events around each of {args.dist_steps} further steps (after the timed region; "
                        "the events' own cost is included)"),
        "hot_ms_per_step": hot,
        "hot_value": round(bench.step_bytes / (hot * 1e-3) / 1e9, 2) if hot else None,
        "hot": ("the same K/V pool every step (no rotation): part of it can stay in the 256 MB Infinity "
                "Cache between steps; reported beside value, never as value"),
        "decode_partition_kernel_ms": round(part_avg_ms, 5),
        "decode_merge_kernel_ms": round(merge_avg_ms, 5),
        "kernel_timing": f"HIP events on the compute stream around {calls} of the {args.steps} timed steps",
        "roofline": roofline,
        "host": platform.node(),
    }
    if getattr(bench, "logical_bytes", None):
        result["logical_GBps"] = round(bench.logical_bytes / step_s / 1e9, 1)
    if getattr(bench, "copy_blocks", None):
        result["copy_blocks"] = bench.copy_blocks
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(bench, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
