"""Build libkvlr.so for gfx950 with hipcc, in-tree.

    python -m decode_attention_rank_amd.build [--jobs N]

Each kernel source compiles to an object under _build/ in parallel; the
objects link into decode_attention_rank_amd/libkvlr.so.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvlr.so")

SOURCES = ["kvlr_api.hip", "k_route.hip", "k_attn.hip", "k_encode.hip", "k_small.hip", "k_oproj.hip",
           "k_fit.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed float32 VALU forms stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the kvlr library needs ROCm's hipcc")


def _compile(src: str) -> tuple[str, float, str]:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    t0 = time.time()
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    # hipcc's host pass warns about the device-only target feature; drop that noise
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in (p.stderr or "").splitlines() if noise not in l)
    return obj, time.time() - t0, warn


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for obj, dt, warn in ex.map(_compile, SOURCES):
            objs.append(obj)
            if verbose:
                print(f"  compiled {os.path.basename(obj)} in {dt:.1f}s", flush=True)
                if warn.strip():
                    print(warn, flush=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"  linked {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    try:
        build(args.jobs)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
