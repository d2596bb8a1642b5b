"""Build the HIP library ``liblinattn.so`` for gfx950 with hipcc.

Every ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in
parallel) and linked into ``gated_delta_rule_27_amd/liblinattn.so``.  The
matrix-core throughput probe that bench.py reports beside the datasheet peak
(``peak/mfma_peak.hip``) is built on its own into ``libmfmapeak.so``, and the
LDS lane-group probe (``peak/lds_banks.hip``) into the executable
``peak/lds_banks``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "liblinattn.so")
PEAK_SRC = os.path.join(HERE, "peak", "mfma_peak.hip")
PEAK_LIB = os.path.join(HERE, "libmfmapeak.so")
LDS_SRC = os.path.join(HERE, "peak", "lds_banks.hip")
LDS_BIN = os.path.join(HERE, "peak", "lds_banks")
ARCH = os.environ.get("LINATTN_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    workers = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "8"))))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                   check=True)
    os.replace(tmp, LIB)
    ptmp = PEAK_LIB + ".tmp"
    r = subprocess.run([HIPCC, *FLAGS, "-shared", "-o", ptmp, PEAK_SRC], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PEAK_SRC}:\n{r.stdout}{r.stderr}")
    os.replace(ptmp, PEAK_LIB)
    ltmp = LDS_BIN + ".tmp"
    r = subprocess.run([HIPCC, *FLAGS, "-o", ltmp, LDS_SRC], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {LDS_SRC}:\n{r.stdout}{r.stderr}")
    os.replace(ltmp, LDS_BIN)
    if verbose:
        print(f"built {LIB}, {PEAK_LIB} and {LDS_BIN}")
    return LIB


if __name__ == "__main__":
    build()
