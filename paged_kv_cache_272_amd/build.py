"""Build libpa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every call compiles from source; the result lands next to this file so it
travels with the source tree.  This script is loaded by file path (it must
work before libpa.so exists, when the package itself cannot be imported).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB_PATH = os.path.join(HERE, "libpa.so")
BUILD_DIR = os.path.join(HERE, "_build")

ARCH = "gfx950"
SOURCES = ["pa_api.hip", "plan.cpp", "block_manager.cpp", "cache_ops.hip", "decode_valu.hip", "decode_mfma.hip",
           "attend_planned.hip", "probes.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed-fp32 instructions anywhere in the library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


ISA_CHECK = os.path.join(HERE, "isa_check.py")


def _check_device_isa(src: str) -> None:
    """Reject generated code that writes through the scalar data cache (the
    opcode list and the scan live in isa_check.py, a build-time-only file
    that copies of the tree sent to a GPU machine leave out; there the scan
    is skipped)."""
    import importlib.util
    if not os.path.exists(ISA_CHECK):
        return
    spec = importlib.util.spec_from_file_location("pa_isa_check", ISA_CHECK)
    isa_check = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(isa_check)
    asm = os.path.join(BUILD_DIR, os.path.basename(src) + ".s")
    cmd = [hipcc(), *HIPCC_FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", asm]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"device assembly failed for {src}:\n{res.stderr}")
    bad = isa_check.scalar_cache_writes(open(asm).read())
    if bad:
        raise RuntimeError(f"{src}: generated code writes through the scalar cache: {bad[0]}")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, 2 * len(SOURCES))) as ex:
        objs_f = [ex.submit(_compile, src) for src in SOURCES]
        checks = [ex.submit(_check_device_isa, src) for src in SOURCES]
        objs = [f.result() for f in objs_f]
        for f in checks:
            f.result()
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        scan = "scanned" if os.path.exists(ISA_CHECK) else "not scanned (isa_check.py absent)"
        print(f"built {LIB_PATH}; device code {scan} for scalar-cache writes")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
