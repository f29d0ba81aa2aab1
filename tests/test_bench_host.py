"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the HBM-traffic
record built from rocprofv3 counter files, and the kernel-source hash that
decides whether a stored record still applies."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def _write_counter_csv(path, counter, rows):
    """rows: (kernel name, value in KiB per dispatch), in rocprofv3's column layout."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    fields = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for i, (name, kib) in enumerate(rows):
            w.writerow({"Correlation_Id": i + 1, "Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": kib})


def test_traffic_record_scales_each_counter_by_the_copy_probe(tmp_path, monkeypatch):
    bench = _bench()
    kernel = "void pa::(anonymous namespace)::decode_mfma_balanced_kernel<128, 0>(pa::DecodeArgs)"
    copy = "pa::(anonymous namespace)::probe_copy_kernel(uint4*, uint4 const*, long)"
    gib_kib = bench.COPY_PROBE_BYTES / 1024.0
    # the read counter sees half of the copy's 1 GiB, the write counter all of it
    _write_counter_csv(str(tmp_path / "fetch" / "run" / "fetch_counter_collection.csv"), "FETCH_SIZE",
                       [(copy, gib_kib / 2), (kernel, 1000.0), (kernel, 1200.0), (kernel, 1100.0),
                        ("__amd_rocclr_copyBuffer", 5.0)])
    _write_counter_csv(str(tmp_path / "write" / "run" / "write_counter_collection.csv"), "WRITE_SIZE",
                       [(copy, gib_kib), (kernel, 10.0), (kernel, 30.0), (kernel, 20.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_file", lambda workload: str(out))
    bench.traffic_record("decode_8b", str(tmp_path / "fetch"), str(tmp_path / "write"))
    rec = json.loads(out.read_text())
    assert rec["read_scale"] == 2.0 and rec["write_scale"] == 1.0
    # medians per dispatch: 1100 KiB read (x2), 20 KiB written (x1)
    assert rec["fetch_bytes_per_launch_raw"] == 1100.0 * 1024
    assert rec["write_bytes_per_launch_raw"] == 20.0 * 1024
    assert rec["hbm_bytes_per_launch"] == round(2 * 1100.0 * 1024 + 20.0 * 1024)
    assert rec["kernel"] == "decode_mfma_balanced_kernel"
    assert rec["kernel_source_hash"] == bench.kernel_source_hash(bench.KERNELS["decode_8b"][1])


def test_source_hash_follows_the_kernel_sources(tmp_path, monkeypatch):
    bench = _bench()
    csrc = tmp_path / "paged_kv_cache_272_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "a.hip").write_text("kernel one")
    (csrc / "b.h").write_text("header")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h1 = bench.kernel_source_hash(["a.hip", "b.h"])
    assert h1 == bench.kernel_source_hash(["a.hip", "b.h"])
    (csrc / "b.h").write_text("header, changed")
    assert bench.kernel_source_hash(["a.hip", "b.h"]) != h1
    # every workload's dominant kernel has a stored source list
    assert set(bench.KERNELS) >= {"decode_8b", "decode_70b", "long_ctx_fp8", "shared_prefix_32x8", "verify4_8b",
                                  "chunked_prefill", "decode_8b_int4"}


def test_cpu_baseline_counts_every_sequence_once_per_call_and_reports_its_threads():
    """The CPU baseline's threads take sequences in turn: every call's bytes
    are counted once, the sequence index cycles over the batch, and `cores`
    is the thread count it ran with."""
    import threading
    import types
    bench = _bench()
    seen, lock = [], threading.Lock()

    def one(b):
        with lock:
            seen.append(b)
        return 1000 + b

    fake = types.SimpleNamespace(cpu_prepare=lambda: None, cpu_one=one, num_seqs=5, cpu_kind="fake")
    rec = bench.cpu_baseline(fake, 0.3, threads=3)
    assert rec["cores"] == 3 and rec["kind"] == "oracle" and rec["value"] > 0
    assert all(0 <= b < 5 for b in seen) and len(seen) >= 5
    # the reported rate is the summed bytes of exactly the calls made (both
    # figures are rounded in the record: 1% covers that)
    elapsed = len(seen) / rec["seqs_per_s"]
    total = sum(1000 + b for b in seen)
    assert abs(rec["value"] * 1e9 * elapsed - total) <= 1e-2 * total
    # sequences are handed out in order, so over any 5 consecutive calls each index appears once
    counts = [seen.count(b) for b in range(5)]
    assert max(counts) - min(counts) <= 1 + 3    # (threads may finish their last call out of order)
