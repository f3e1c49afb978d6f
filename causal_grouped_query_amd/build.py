"""Build libgqa_attn.so in-tree with hipcc for gfx950.

Every .hip file under csrc/ is compiled to an object in parallel and linked
into causal_grouped_query_amd/libgqa_attn.so; the measurement probes under
probes/ (peak MFMA and streaming-copy rates for the benchmark's roofline
context) go into libgqa_probes.so.  Device code is built with the
packed-fp32 instructions disabled.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgqa_attn.so")
# debug build of the same library: LDS buffers and the split-KV workspace are
# filled with NaN before use (GQA_DEBUG_NANFILL), so a read of anything no
# copy or kernel wrote shows up in the results; select it with GQA_ATTN_LIB
NANFILL_LIB = os.path.join(PKG, "libgqa_attn_nanfill.so")
PROBE_LIB = os.path.join(PKG, "libgqa_probes.so")  # measurement aids for bench.py (not the attention ABI)
OBJDIR = os.path.join(PKG, "_build")
ARCH = os.environ.get("GQA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str, variant: str = "") -> str:
    sub = "probe_" if os.path.basename(os.path.dirname(src)) == "probes" else variant
    obj = os.path.join(OBJDIR, sub + os.path.basename(src).replace(".hip", ".o"))
    extra = ["-DGQA_DEBUG_NANFILL=1"] if variant == "nanfill_" else []
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probe_srcs = sorted(glob.glob(os.path.join(PKG, "probes", "*.hip")))
    jobs = [(s, "") for s in srcs + probe_srcs] + [(s, "nanfill_") for s in srcs]
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    n, m = len(srcs), len(probe_srcs)
    _link(objs[:n], LIB)
    _link(objs[n:n + m], PROBE_LIB)
    _link(objs[n + m:], NANFILL_LIB)
    if verbose:
        print(f"built {LIB}, {PROBE_LIB} and {NANFILL_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
