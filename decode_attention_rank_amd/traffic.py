"""Measured HBM traffic and instruction counters of one kernel from rocprofv3
counter runs.

    # a copy-shaped kernel of known size, to scale the counters
    python -m decode_attention_rank_amd.traffic copy --mib 1024 --reps 4
    # after one FETCH_SIZE run and one WRITE_SIZE run each of the bench and of the copy:
    python -m decode_attention_rank_amd.traffic summarize --kernel route_kernel \
        --workload llama3-8b-routed-32k --fetch DIR --write DIR \
        --copy-fetch DIR --copy-write DIR --copy-mib 1024 --algo-bytes N --out FILE

    # after one run with the shader-sequencer counters below (SQ_COUNTERS):
    python -m decode_attention_rank_amd.traffic counters --kernel route_kernel \
        --workload llama3-8b-routed-32k --dir DIR [--build-tag valu] --out FILE

FETCH_SIZE and WRITE_SIZE are the L2's reads from and writes to memory, in
KiB per dispatch. The copy (y = -x over float32, each byte read once and
written once) tells how many real bytes one counted KiB stands for; the
kernel's counts are scaled by that factor. The record carries the hash of the
kernel's source so that a stale record is ignored.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = {
    "route_kernel": os.path.join(ROOT, "decode_attention_rank_amd", "csrc", "k_route.hip"),
    "attn_kernel": os.path.join(ROOT, "decode_attention_rank_amd", "csrc", "k_attn.hip"),
    "encode_kernel": os.path.join(ROOT, "decode_attention_rank_amd", "csrc", "k_encode.hip"),
    "moments_mfma_kernel": os.path.join(ROOT, "decode_attention_rank_amd", "csrc", "k_fit.hip"),
}
SOURCES["merge_kernel"] = SOURCES["attn_kernel"]
SOURCES["select_kernel"] = SOURCES["route_kernel"]
COPY_KERNEL_HINT = "neg_kernel"

# one rocprofv3 pass: eight shader-sequencer counters and the GPU-active clock
SQ_COUNTERS = ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
               "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU",
               "SQ_INSTS_LDS", "SQ_WAVES", "GRBM_GUI_ACTIVE"]
# MI355X: 256 compute units of 4 SIMDs each, in 8 XCDs (one GRBM_GUI_ACTIVE
# instance per XCD; rocprofv3's per-dispatch value is their sum)
CU_NUM, SIMD_NUM, XCD_NUM = 256, 1024, 8


def source_hash(path: str) -> str:
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def run_copy(mib: int, reps: int) -> None:
    import torch
    n = mib * (1 << 20) // 4
    x = torch.randn(n, device="cuda", dtype=torch.float32)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(f"copy: {reps} x neg over {mib} MiB float32 (read {mib} MiB, write {mib} MiB)", flush=True)


def _counter_rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    for f in files:
        with open(f) as fh:
            yield from csv.DictReader(fh)


def per_dispatch(d: str, counter: str, name_part: str):
    """Counter value per dispatch of the kernels whose name contains name_part."""
    vals = {}
    for r in _counter_rows(d):
        if r.get("Counter_Name") != counter or name_part not in r.get("Kernel_Name", ""):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for a kernel named *{name_part}* under {d}")
    return list(vals.values())


def table(d: str, counter: str, name_part: str = "kvlr") -> list:
    """(kernel, dispatches, median value) for every kernel whose name contains name_part."""
    per = {}
    for r in _counter_rows(d):
        if r.get("Counter_Name") != counter or name_part not in r.get("Kernel_Name", ""):
            continue
        k = r["Kernel_Name"]
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        per.setdefault(k, {})
        per[k][key] = per[k].get(key, 0.0) + float(r["Counter_Value"])
    return [(k, len(v), statistics.median(v.values())) for k, v in sorted(per.items())]


def summarize(a) -> dict:
    copy_bytes = a.copy_mib * (1 << 20)
    cf = statistics.median(per_dispatch(a.copy_fetch, "FETCH_SIZE", COPY_KERNEL_HINT))
    cw = statistics.median(per_dispatch(a.copy_write, "WRITE_SIZE", COPY_KERNEL_HINT))
    kf = per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    kw = per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    fetch_b = statistics.median(kf) * 1024.0 * f_scale
    write_b = statistics.median(kw) * 1024.0 * w_scale
    rec = {
        "kernel": a.kernel, "workload": a.workload,
        "dispatches": {"fetch": len(kf), "write": len(kw)},
        "fetch_kib_median": statistics.median(kf), "write_kib_median": statistics.median(kw),
        "copy_bytes_each_way": copy_bytes,
        "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "hbm_read_bytes_per_launch": int(fetch_b), "hbm_write_bytes_per_launch": int(write_b),
        "hbm_bytes_per_launch": int(fetch_b + write_b),
        "algo_bytes_per_launch": a.algo_bytes,
        "traffic_over_algo": round((fetch_b + write_b) / a.algo_bytes, 4) if a.algo_bytes else None,
        "source_sha256_16": source_hash(SOURCES[a.kernel]),
    }
    return rec


def counters(a) -> dict:
    """Median per dispatch of each SQ_COUNTERS value, and the derived shares
    rocprofv3 defines: MfmaUtil = MFMA busy cycles over (GPU-active cycles x
    SIMDs), VALUBusy = VALU-active wave cycles over (GPU-active cycles x CUs)."""
    med = {c: statistics.median(per_dispatch(a.dir, c, a.kernel)) for c in SQ_COUNTERS}
    n = len(per_dispatch(a.dir, "SQ_WAVES", a.kernel))
    gui = med["GRBM_GUI_ACTIVE"] / XCD_NUM  # cycles of one XCD
    rec = {
        "kernel": a.kernel, "workload": a.workload, "build": a.build_tag, "dispatches": n,
        "median_per_dispatch": {c: med[c] for c in SQ_COUNTERS},
        "gpu_active_cycles": round(gui, 1),
        "mfma_busy_pct": round(100.0 * med["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * SIMD_NUM), 3)
        if gui else None,
        "valu_busy_pct": round(100.0 * med["SQ_ACTIVE_INST_VALU"] / CU_NUM / gui, 3) if gui else None,
        "mfma_flop": med["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 + med["SQ_INSTS_VALU_MFMA_MOPS_F32"] * 512,
        "valu_insts_per_wave": round(med["SQ_INSTS_VALU"] / med["SQ_WAVES"], 1)
        if med["SQ_WAVES"] else None,
        "mfma_insts_per_wave": round(med["SQ_INSTS_MFMA"] / med["SQ_WAVES"], 1)
        if med["SQ_WAVES"] else None,
        "source_sha256_16": source_hash(SOURCES[a.kernel]),
    }
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=4)
    s = sub.add_parser("summarize")
    s.add_argument("--kernel", required=True, choices=sorted(SOURCES))
    s.add_argument("--workload", required=True)
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--copy-fetch", required=True)
    s.add_argument("--copy-write", required=True)
    s.add_argument("--copy-mib", type=int, default=1024)
    s.add_argument("--algo-bytes", type=int, required=True)
    s.add_argument("--out", required=True)
    q = sub.add_parser("counters")
    q.add_argument("--kernel", required=True, choices=sorted(SOURCES))
    q.add_argument("--workload", required=True)
    q.add_argument("--dir", required=True)
    q.add_argument("--build-tag", default="default")
    q.add_argument("--out", required=True)
    t = sub.add_parser("table")
    t.add_argument("--dir", required=True)
    t.add_argument("--counter", required=True)
    t.add_argument("--name", default="kvlr")
    a = ap.parse_args(argv)
    if a.cmd == "copy":
        run_copy(a.mib, a.reps)
        return
    if a.cmd == "table":
        for k, n, v in table(a.dir, a.counter, a.name):
            print(f"{a.counter}\t{n}\t{v:.1f}\t{k}")
        return
    rec = summarize(a) if a.cmd == "summarize" else counters(a)
    with open(a.out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    json.dump(rec, sys.stdout)
    print()


if __name__ == "__main__":
    main()
