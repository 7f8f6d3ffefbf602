"""Build the gfx950 HIP library ``libattn_bwd.so`` in-tree.

Every ``csrc/*.hip`` file is compiled to an object under ``_build/`` (in
parallel) and linked into ``atomics_bwd_preprocess_amd/libattn_bwd.so``.
``microbench/atomic_rate.hip`` (the atomic-rate measurement the benchmark
script runs; not part of the attention ABI) is linked into
``libattn_microbench.so`` beside it.
Run ``python -m atomics_bwd_preprocess_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libattn_bwd.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
MICROBENCH_SRC = os.path.join(PKG_DIR, "microbench", "atomic_rate.hip")
MICROBENCH_LIB = os.path.join(PKG_DIR, "libattn_microbench.so")
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled for every device compile.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _filter(text: str) -> str:
    # hipcc's host pass does not know the packed-fp32 feature; that warning is noise.
    return "\n".join(ln for ln in text.splitlines()
                     if "packed-fp32-ops" not in ln and ln.strip() != "1 warning generated.")


def _compile(hipcc: str, src: str, obj: str, extra: list) -> None:
    cmd = [hipcc, *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = _filter(r.stdout + r.stderr)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)


def sources() -> list:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _link(hipcc: str, objs: list, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, extra_flags: list | None = None) -> str:
    """Compile and link the library (and the microbenchmark library); returns
    the library's path.  Always rebuilds."""
    hipcc = _hipcc()
    extra = list(extra_flags or [])
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources() + [MICROBENCH_SRC]
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda so: _compile(hipcc, so[0], so[1], extra), zip(srcs, objs)))
    _link(hipcc, objs[:-1], LIB_PATH)
    _link(hipcc, objs[-1:], MICROBENCH_LIB)
    if verbose:
        print(f"built {LIB_PATH} and {MICROBENCH_LIB}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
