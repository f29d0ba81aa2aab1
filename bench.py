#!/usr/bin/env python3
"""Paged-KV decode benchmark on one MI355X.

One step = one decode step of the Llama-3-8B-shaped layer (64 sequences,
32 query / 8 KV heads, head_dim 128, bf16, contexts U{128..4096}): each
sequence's new token is written into its slot and the paged decode runs
over the cache including it.  By default this is one pa_decode_append call
(the decode kernel writes the new rows itself, then the log-sum-exp merge
kernel runs); `--step separate` times pa_cache_write + pa_decode instead.  Inputs are seeded,
synthetic and resident in HBM before timing; the K/V pool is rotated over
several copies so the 256 MB Infinity Cache cannot hold it between steps.

Prints one JSON line: whole-step KV throughput (algorithmic bytes / step
time), sequences/s, fraction of the 8 TB/s HBM spec and of a measured
stream-read ceiling, the decode partition kernel's roofline entry (its
algorithmic bytes over its average duration, from HIP events recorded on
its own stream during the timed steps), and the CPU oracle timed on a
bounded sample of the same workload.
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic_llama3_8b_bs64.json")
KERNEL_SOURCES = ["decode_valu.hip", "decode_mfma.hip", "pa_api.hip", "pa_device.h", "pa_internal.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
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
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--pools", type=int, default=3, help="K/V pool copies rotated across steps")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
DECODE_KERNEL = "decode_mfma_balanced_kernel"
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


def traffic_record(fetch_dir, write_dir):
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
    dec_read, dec_write = pick(fetch, DECODE_KERNEL), pick(write, DECODE_KERNEL)
    rec = {
        "kernel": DECODE_KERNEL,
        "kernel_source_hash": kernel_source_hash(),
        "fetch_bytes_per_launch_raw": dec_read, "write_bytes_per_launch_raw": dec_write,
        "copy_probe_bytes": COPY_PROBE_BYTES, "copy_probe_fetch_raw": copy_read, "copy_probe_write_raw": copy_write,
        "read_scale": read_scale, "write_scale": write_scale,
        "hbm_bytes_per_launch": round(dec_read * read_scale + dec_write * write_scale),
        "method": "rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (separate runs) over bench.py; median "
                  "per-dispatch value, each scaled by (known bytes / counter) of a 1 GiB probe copy in the "
                  "same run",
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def cpu_baseline(wl, k_ref, v_ref, budget_s):
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        done, t_start = [], time.perf_counter()
        while time.perf_counter() - t_start < budget_s:       # whole passes over the batch, as time allows
            for b in range(wl.num_seqs):
                oracle.decode_ref(wl.q, k_ref, v_ref, wl.block_tables, wl.context_lens, wl.scale, "bf16",
                                  "bf16", seqs=[b])
                done.append(b)
                if time.perf_counter() - t_start >= budget_s:
                    break
        elapsed = time.perf_counter() - t_start
    lens = wl.context_lens[done]
    nbytes = oracle.decode_algorithmic_bytes(lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, 2, 2, 2)
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": round(nbytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"float64 numpy oracle (decode_ref), BLAS limited to 1 thread, {len(done)} sequence decodes "
                  f"cycling over the {wl.num_seqs}-sequence batch ({int(lens.sum())} tokens, "
                  f"{nbytes / 1e6:.1f} MB algorithmic) in {elapsed:.1f} s; host CPU {cpu}",
        "seqs_per_s": round(len(done) / elapsed, 3),
    }


def main():
    args = parse_args()
    if args.traffic_from:
        traffic_record(*args.traffic_from)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the decode shards by sequence or KV head with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_272_amd as pa
    import pa_workloads as W

    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    wl = W.config2()
    gen_s = time.perf_counter() - t_gen
    print(f"# workload generated in {gen_s:.1f} s: {wl.num_blocks} blocks, sum ctx {int(wl.context_lens.sum())}",
          file=sys.stderr, flush=True)

    def dev(a, bf16=False):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if bf16 else torch.from_numpy(a)
        return t.to("cuda")

    q = dev(wl.q, True)
    new_k, new_v = dev(wl.new_k, True), dev(wl.new_v, True)
    bt, cl, slots = dev(wl.block_tables), dev(wl.context_lens), dev(wl.slot_mapping)
    k0, v0 = dev(wl.k_cache, True), dev(wl.v_cache, True)
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(args.pools - 1)]
    out = torch.empty_like(q)
    part = pa.pa_decode_partition_tokens(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                         wl.max_context_len, args.partition_tokens)
    ws_bytes = pa.pa_decode_workspace_size(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                           wl.max_context_len, args.partition_tokens)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    steps = []
    for kc, vc in pools:
        if args.step == "append":
            steps.append((pa.prepare_decode_append(out, q, new_k, new_v, kc, vc, bt, cl, wl.max_context_len,
                                                   wl.scale, partition_tokens=args.partition_tokens,
                                                   workspace=ws),))
        else:
            steps.append((pa.prepare_cache_write(new_k, new_v, kc, vc, slots),
                          pa.prepare_decode(out, q, kc, vc, bt, cl, wl.max_context_len, wl.scale,
                                            partition_tokens=args.partition_tokens, workspace=ws)))

    import oracle
    decode_bytes = oracle.decode_algorithmic_bytes(wl.context_lens, wl.num_q_heads, wl.num_kv_heads,
                                                   wl.head_dim, 2, 2, 2)
    write_bytes = wl.num_seqs * wl.num_kv_heads * wl.head_dim * 2 * 2 * 2 + wl.num_seqs * 8
    step_bytes = decode_bytes + write_bytes

    copy_probe(pa, torch)
    peak_meas = measured_stream_read(pa, torch)
    print(f"# measured stream read {peak_meas:.0f} GB/s", file=sys.stderr, flush=True)

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
    value = step_bytes / step_s / 1e9
    part_avg_ms = part_ms / max(calls, 1)
    merge_avg_ms = merge_ms / max(calls, 1)
    achieved = decode_bytes / (part_avg_ms * 1e-3) / 1e9

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("kernel_source_hash") == kernel_source_hash():
            traffic = rec.get("hbm_bytes_per_launch")

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
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)*0.5 bf16 q/K/V, shuffled 16-token block pool)",
        "config": {
            "workload": "llama3_8b_shape_decode_bs64",
            "batch": wl.num_seqs, "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads,
            "head_dim": wl.head_dim, "block_size": 16, "context_lens": "U{128..4096}",
            "sum_context": int(wl.context_lens.sum()), "kv_dtype": "bf16", "pool_blocks": wl.num_blocks,
            "pools_rotated": len(pools),
            "work_split": ("balanced slices of the (sequence, block) list" if args.partition_tokens == 0
                           else f"{part}-token partitions"),
            "step": ("pa_decode_append: slot write of the 64 new tokens fused into the decode"
                     if args.step == "append" else "pa_cache_write(64 tokens) + pa_decode"),
        },
        "seqs_per_s": round(wl.num_seqs / step_s, 1),
        "pct_of_spec_hbm": round(100 * value / SPEC_HBM_GBPS, 2),
        "measured_stream_read_GBps": round(peak_meas, 1),
        "pct_of_measured_stream_read": round(100 * value / peak_meas, 2),
        "step_algorithmic_bytes": int(step_bytes),
        "decode_partition_kernel_ms": round(part_avg_ms, 5),
        "decode_merge_kernel_ms": round(merge_avg_ms, 5),
        "kernel_timing": f"HIP events on the decode stream around {calls} of the {args.steps} timed steps",
        "roofline": {
            "kernel": "decode partition kernel",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": SPEC_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / SPEC_HBM_GBPS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": int(decode_bytes),
        },
        "host": platform.node(),
    }
    if not args.no_cpu_baseline:
        k_ref, v_ref = oracle.cache_write_ref(wl.k_cache, wl.v_cache, wl.new_k, wl.new_v, wl.slot_mapping,
                                              "bf16", "bf16")
        result["cpu_baseline"] = cpu_baseline(wl, k_ref, v_ref, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
