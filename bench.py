"""Decode-attention throughput over a low-rank compressed, paged KV cache.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

One step = the whole decode hot path for one layer of one GPU's head share:
append-encode of each sequence's new token(s), query projection, page routing
(routed workloads), attention over the chosen pages, and the up-projection.
Inputs are seeded synthetic caches already resident in HBM. Prints one JSON
line: KV-tokens/s (sum of context lengths / step time), the roofline of the
dominant kernel (timed live with HIP events on its own stream), and the CPU
oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from decode_attention_rank_amd.session import DecodeSession  # noqa: E402
from decode_attention_rank_amd.traffic import source_hash  # noqa: E402
from decode_attention_rank_amd.workloads import DEFAULT_BENCH_WORKLOAD, WORKLOADS  # noqa: E402

METRIC = "decode-attn KV-tokens/s over compressed cache + % of HBM peak GB/s (1 GPU)"
HBM_PEAK_GBPS = 8000.0
CPU_CACHE_BYTES = 6 << 30  # host memory for oracle inputs repeated after the first pass
ROUTE_SOURCE = os.path.join(ROOT, "decode_attention_rank_amd", "csrc", "k_route.hip")
ATTN_SOURCE = os.path.join(ROOT, "decode_attention_rank_amd", "csrc", "k_attn.hip")
FIT_SOURCE = os.path.join(ROOT, "decode_attention_rank_amd", "csrc", "k_fit.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(kernel: str, workload: str, src: str):
    """HBM bytes per launch from a committed counter summary, if it is current."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256_16") != source_hash(src):
        return None  # kernel changed since the counters were taken
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(sess, budget_s: float):
    """The oracle as it stands, on whole (sequence, KV head) pairs until the
    time budget is spent; rate scaled to KV-tokens/s of the full step."""
    import numpy as np
    from threadpoolctl import threadpool_info

    wl = sess.wl
    seqs = list(range(wl.batch))
    np.random.default_rng(0).shuffle(seqs)
    order = [(b, g) for b in seqs for g in range(wl.num_kv_heads)]
    memo = {}
    spent, tokens, pairs, passes = 0.0, 0, 0, 0
    cache, cached_bytes = [], 0
    while spent < budget_s:
        passes += 1
        items = cache if passes > 1 else (_oracle_inputs(sess, b, g, memo) for b, g in order)
        for item in items:
            t0 = time.perf_counter()
            _oracle_pair(wl, sess.scale, item)
            spent += time.perf_counter() - t0
            tokens += item["L"]
            pairs += 1
            if passes == 1 and cached_bytes < CPU_CACHE_BYTES:
                cache.append(item)
                cached_bytes += sum(a.nbytes for a in item["prefix"].values())
            if spent >= budget_s:
                break
        if not cache:
            break
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    value = tokens / wl.num_kv_heads / spent
    return {
        "value": value, "unit": "KV-tokens/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"{pairs} (sequence, KV head) pair runs, {passes} pass(es) over the "
                   f"{wl.batch * wl.num_kv_heads} pairs taken sequence by sequence in shuffled "
                   f"order (later passes repeat the first {len(cache)}), {tokens} context "
                   f"tokens, {spent:.1f} s of float64 numpy on the host; "
                   f"rate = tokens / H_kv / seconds"),
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def _oracle_inputs(sess, b, g, memo):
    """One pair's inputs for the oracle, in float64 (not timed)."""
    from tests import gpu_harness as H

    if memo.get("b") != b:
        memo.clear()
        memo["b"], memo["rows"] = b, sess.prefix_rows(b)
    st_rows = memo["rows"]
    off = sum(sess.n_new[:b])
    n = sess.n_new[b]
    prefix = {k: H.f64(v[g]) for k, v in st_rows.items()}
    prefix["k_lat"] = H.k_cols(sess, g, prefix["k_lat"])  # the head's kept residual coordinates
    return {
        "prefix": prefix,
        "L_before": sess.lens_before[b], "L": sess.seq_lens[b],
        "K": H.f64(sess.k_new[off:off + n, g]), "V": H.f64(sess.v_new[off:off + n, g]),
        "f": H.factors_np(sess, g), "q": H.q_group(sess, b, g),
    }


def _oracle_pair(wl, scale, it):
    """Append, route, attend and up-project one pair with the oracle."""
    import oracle as O

    f = it["f"]
    st = O.append_tokens(it["prefix"], it["L_before"], it["K"], it["V"], f["A_v"], f["A_k"],
                         f["W_pred"], key_mode=wl.key_mode, storage=wl.lat_storage)
    res = O.decode_pair(it["q"], st, f, it["L"], wl.page_size, key_mode=wl.key_mode, scale=scale,
                        topk=(wl.topk_num, wl.topk_den))
    O.upproject(res["z"], f["B_v"])


def time_output_projection(sess, reps: int = 50):
    """The folded output projection F . z (F = W_o blockdiag(B_v^T)), timed on
    its own after the steps: it reads F ([hidden][H_q r_v] bf16) once."""
    sess.prepare_output_projection()
    stream = torch.cuda.current_stream()
    for _ in range(5):
        sess.output_projection()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        sess.output_projection()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    wl = sess.wl
    f_bytes = sess.F.numel() * sess.F.element_size()
    w_bytes = sess.W_o.numel() * sess.W_o.element_size()
    gbps = f_bytes / (us * 1e-6) / 1e9
    return {"kernel": "oproj_kernel", "hidden": sess.hidden, "avg_launch_us": round(us, 2),
            "folded_weight_bytes": f_bytes, "unfolded_weight_bytes": w_bytes,
            "achieved_gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}


def time_factor_fit(reps: int = 10):
    """The factor fit on its calibration workload: the GPU moments call
    (moments_mfma_kernel plus the fixed-order float64 sum of its per-run
    partials) timed with HIP events, and the whole synchronous
    kvlr_fit_factors call (moments, copy to host, float64 eigen-solves,
    factor writes) by wall clock."""
    from decode_attention_rank_amd import synth
    from decode_attention_rank_amd.fit import FactorFit
    from decode_attention_rank_amd.workloads import DEFAULT_FIT_WORKLOAD, FIT_WORKLOADS

    wl = FIT_WORKLOADS[DEFAULT_FIT_WORKLOAD]
    n = synth.fit_sample_count(wl)
    H, d = wl.num_kv_heads, wl.head_dim
    k, v = synth.make_fit_samples(wl, n, device="cuda")
    fit = FactorFit(wl, n)
    moments = torch.empty(H, 3, d, d, dtype=torch.float64, device="cuda")
    stream = torch.cuda.current_stream()
    fit.fit(k, v)
    for _ in range(3):
        fit.moments(k, v, n, moments, 0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fit.moments(k, v, n, moments, 0)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    t0 = time.perf_counter()
    for _ in range(3):
        fit.fit(k, v)
    fit_ms = (time.perf_counter() - t0) * 1e3 / 3
    kernel_algo = 2 * n * H * d * k.element_size()   # the samples, read once
    algo = kernel_algo + H * 3 * d * d * 8             # plus the float64 moments written
    flops = 2.0 * n * H * 3 * d * d
    gbps = algo / (us * 1e-6) / 1e9
    del k, v
    return {"workload": wl.name, "samples_per_kv_head": n, "num_kv_heads": H, "head_dim": d,
            "rank_v": wl.rank_v, "rank_k": wl.rank_k, "storage": wl.storage,
            "timed": "kvlr_fit_moments: moments_mfma_kernel + moments_sum_kernel",
            "moments_call_us": round(us, 2), "algo_bytes_per_call": algo,
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                         "traffic": measured_traffic("moments_mfma_kernel", wl.name, FIT_SOURCE),
                         "kernel": "moments_mfma_kernel", "kernel_algo_bytes": kernel_algo},
            "mfma_tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "fit_factors_call_ms": round(fit_ms, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_BENCH_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fit", action="store_true", help="skip the factor-fit measurement")
    ap.add_argument("--fused", action="store_true",
                    help="up-projection inside the attention launch instead of its own")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    wl = WORKLOADS[args.workload]
    log(f"[bench] staging workload {wl.name}")
    t0 = time.time()
    sess = DecodeSession(wl, "cuda")
    torch.cuda.synchronize()
    log(f"[bench] staged in {time.time() - t0:.1f}s; KV tokens/step {sess.kv_tokens()}")

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]

    attend = sess.attend_upproject if args.fused and wl.value_basis != "identity" else sess.attend

    def step(i=None):
        sess.prepare()
        if wl.routed:
            if i is not None:
                ev[i][0].record(stream)
            sess.route()
            if i is not None:
                ev[i][1].record(stream)
            attend()
        else:
            if i is not None:
                ev[i][0].record(stream)
            attend()
            if i is not None:
                ev[i][1].record(stream)
        if not args.fused and wl.value_basis != "identity":
            sess.upproject()  # the uncompressed reference stores values as they are: o = z

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    log(f"[bench] timed {args.steps} steps in {elapsed:.3f}s")

    ms_per_step = elapsed * 1e3 / args.steps
    value = sess.kv_tokens() * args.steps / elapsed
    dom_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    if wl.routed:
        dom_bytes = sess.route_bytes()
        dom_name = "route_kernel"
        dom_src = ROUTE_SOURCE
    else:
        dom_bytes = sess.attend_bytes()
        dom_name = "attn_kernel"
        dom_src = ATTN_SOURCE
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    step_bytes = sess.append_bytes() + (sess.route_bytes() if wl.routed else 0) + sess.attend_bytes()
    roof = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": measured_traffic(dom_name, wl.name, dom_src),
        "kernel": dom_name, "algo_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_ms * 1e3, 2),
    }
    cfg = {
        "workload": wl.name, "batch": wl.batch, "context": (sum(sess.seq_lens) // wl.batch),
        "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
        "page_size": wl.page_size, "rank_v": wl.rank_v, "rank_k": wl.rank_k,
        "storage": wl.storage, "keys": wl.key_mode,
        "topk": f"{wl.topk_num}/{wl.topk_den}" if wl.routed else "all",
        "append_per_seq": wl.append_per_seq, "parallelism": "single-gpu",
    }
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "KV-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "config": cfg,
        "step_algo_bytes": step_bytes,
        "kernel_algo_bytes": {"encode_kernel": sess.append_bytes(), "attn_kernel": sess.attend_bytes(),
                              "route_kernel": sess.route_bytes() if wl.routed else 0},
        "step_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": roof,
    }
    if wl.storage == "bf16":
        out["output_projection"] = time_output_projection(sess)
    if not args.no_fit:
        log("[bench] timing the factor fit")
        out["factor_fit"] = time_factor_fit()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(sess, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
