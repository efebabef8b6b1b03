"""Build libkvlr.so for gfx950 with hipcc, in-tree.

    python -m decode_attention_rank_amd.build [--jobs N]
    # a variant with compile-time switches, e.g. vector-ALU scoring:
    python -m decode_attention_rank_amd.build -D KVLR_ROUTE_MFMA=0 -D KVLR_ATTN_MFMA=0 \
        --out /tmp/libkvlr_valu.so

Each kernel source compiles to an object under _build/ in parallel (the
plain C++ host source with the host compiler only); the objects link into
decode_attention_rank_amd/libkvlr.so. A variant's objects go
to a folder of their own under _build/ and its library to --out; the binding
loads it when KVLR_LIBRARY names it.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
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
           "k_fit.hip", "k_outfit.hip", "kvlr_host_solve.cpp"]

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


# plain C++ host sources (no device code): the host compiler alone
HOST_FLAGS = ["-x", "c++", "-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{CSRC}"]


def _compile(src: str, build_dir: str = BUILD, defines: tuple = ()) -> tuple[str, float, str]:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    flags = HOST_FLAGS if src.endswith(".cpp") else FLAGS
    cmd = [hipcc(), *flags, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    t0 = time.time()
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    # hipcc's host pass warns about the device-only target feature; drop that noise
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in (p.stderr or "").splitlines() if noise not in l)
    return obj, time.time() - t0, warn


def build(jobs: int | None = None, verbose: bool = True, defines: tuple = (),
          out: str | None = None) -> str:
    defines = tuple(defines)
    build_dir = BUILD
    if defines:
        tag = hashlib.sha256(" ".join(defines).encode()).hexdigest()[:10]
        build_dir = os.path.join(BUILD, f"variant_{tag}")
    lib_path = out or LIB
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for obj, dt, warn in ex.map(lambda s: _compile(s, build_dir, defines), SOURCES):
            objs.append(obj)
            if verbose:
                print(f"  compiled {os.path.basename(obj)} in {dt:.1f}s", flush=True)
                if warn.strip():
                    print(warn, flush=True)
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"  linked {lib_path}" + (f" with {' '.join(defines)}" if defines else ""), flush=True)
    return lib_path


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-D", dest="defines", action="append", default=[],
                    help="compile-time switch NAME=VALUE for every source (a variant build)")
    ap.add_argument("--out", default=None, help="library path (default: the package's libkvlr.so)")
    args = ap.parse_args()
    if args.defines and not args.out:
        ap.error("a variant build (-D) needs --out, so the package's library stays the default one")
    try:
        build(args.jobs, defines=args.defines, out=args.out)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
