"""Build libdap.so (gfx950) in-tree with hipcc.

    python -m video_dit_mixed_amd.build            # compile every source, link the library

Each .hip file is compiled for gfx950 only; the shared library lands next to this file, and so
does `lds_feed_bench`, a stand-alone timing program for matrix-core products fed from LDS
(`python bench.py --lds-feed` runs it).
Packed-fp32 instruction selection is disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdap.so")
LDS_FEED_BENCH = os.path.join(HERE, "lds_feed_bench")

SOURCES = ["dap_capi.hip", "dap_prep.hip", "dap_draft.hip", "dap_rank.hip", "dap_attn.hip",
           "dap_restore.hip", "dap_stage.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 6)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    cmd = [HIPCC, *[f for f in FLAGS if f != "-fPIC"], os.path.join(CSRC, "lds_feed_bench.hip"),
           "-o", LDS_FEED_BENCH + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for lds_feed_bench.hip:\n{r.stderr}")
    os.replace(LDS_FEED_BENCH + ".tmp", LDS_FEED_BENCH)
    if verbose:
        print(f"built {LIB} and {LDS_FEED_BENCH}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
