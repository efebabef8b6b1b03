"""Decode-attention throughput over a low-rank compressed, paged KV cache.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

One step = the whole decode hot path for one layer of one GPU's head share:
append-encode of each sequence's new token(s) with the query projection in
the same launch, page routing with top-k (routed workloads), attention over
the chosen pages, and the up-projection. Inputs are seeded synthetic caches
already resident in HBM; the step's four launches are replayed as one HIP
graph.

Prints one JSON line:
  * value / ms_per_step: KV-tokens/s (sum of context lengths / step time) of
    the headline workload, from the wall clock around K graph replays
    between two synchronisations;
  * step_time_us: per-step HIP-event times (median, p10, p90), once warm and
    once with a 1 GiB fill between steps (outside the events) so that each
    step starts with the 256 MB Infinity Cache holding none of its inputs;
  * kernels: each launch of the step timed with HIP events on the stream it
    runs on (an eager pass), with its algorithmic bytes;
  * roofline: the dominant kernel (routing, or attention without routing);
  * workloads: the same record for the other configurations (dense 8B,
    70B head share at 128k, mixed append + ragged decode);
  * cpu_baseline: the oracle timed on the host on a bounded sample, and, in
    the same leg, the page sets and outputs of the timed step checked against
    the oracle on every (sequence, KV head) pair of the first pass.
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

from decode_attention_rank_amd import synth  # noqa: E402
from decode_attention_rank_amd.session import DecodeSession  # noqa: E402
from decode_attention_rank_amd.traffic import source_hash  # noqa: E402
from decode_attention_rank_amd.workloads import DEFAULT_BENCH_WORKLOAD, WORKLOADS  # noqa: E402

METRIC = "decode-attn KV-tokens/s over compressed cache + % of HBM peak GB/s (1 GPU)"
HBM_PEAK_GBPS = 8000.0
FLUSH_BYTES = 1 << 30   # written between steps of the cold pass (> the 256 MB Infinity Cache)
CPU_CACHE_BYTES = 6 << 30  # host memory for oracle inputs repeated after the first pass
JOINT_SAMPLES = 8192       # calibration samples of the joint decoder fit
CSRC = os.path.join(ROOT, "decode_attention_rank_amd", "csrc")
KERNEL_SOURCES = {
    "route_kernel": os.path.join(CSRC, "k_route.hip"),
    "select_kernel": os.path.join(CSRC, "k_route.hip"),
    "attn_kernel": os.path.join(CSRC, "k_attn.hip"),
    "encode_kernel": os.path.join(CSRC, "k_encode.hip"),
    "moments_mfma_kernel": os.path.join(CSRC, "k_fit.hip"),
}
# the other configurations reported beside the headline one
OTHER_WORKLOADS = ["llama3-8b-dense-32k", "llama3-70b-share-routed-128k", "mixed-append-routed-ragged"]
VARIANT_WORKLOADS = ["llama3-8b-uncompressed-32k", "llama3-8b-routed-fp8-32k",
                     "llama3-70b-share-routed-fp8-128k", "llama3-8b-routed-adaptive-32k"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed counter summary, if it is current."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None  # kernel changed since the counters were taken
    return rec.get("hbm_bytes_per_launch")


def measured_counters(kernel: str, workload: str):
    """MFMA and VALU busy shares from a committed counter summary, if current."""
    p = os.path.join(ROOT, "profiles", f"counters_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return {"mfma_busy_pct": rec.get("mfma_busy_pct"), "valu_busy_pct": rec.get("valu_busy_pct")}


def pct(xs, q):
    """q-th percentile (0..100) of xs by linear interpolation."""
    s = sorted(xs)
    if not s:
        return None
    x = (len(s) - 1) * q / 100.0
    i = int(x)
    j = min(i + 1, len(s) - 1)
    return s[i] + (s[j] - s[i]) * (x - i)


def spread(us):
    return {"median": round(pct(us, 50), 2), "p10": round(pct(us, 10), 2),
            "p90": round(pct(us, 90), 2), "mean": round(sum(us) / len(us), 2), "n": len(us)}


def step_bytes(sess) -> dict:
    wl = sess.wl
    out = {"encode_kernel": sess.append_bytes(), "attn_kernel": sess.attend_bytes()}
    if wl.routed:
        out["route_kernel"] = sess.route_bytes()
    return out


def measure(sess, steps: int, warmup: int, graph: bool, fused: bool, flush) -> dict:
    """Wall-clock, per-step event and per-kernel event timing of one workload."""
    wl = sess.wl
    stream = torch.cuda.current_stream()
    if graph:
        g = sess.capture(fused=fused)
        run = g.replay
    else:
        g = None
        def run():
            sess.step(fused=fused)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()

    # wall clock around K steps (the headline value)
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0

    def event_pass(with_flush: bool):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i in range(steps):
            if with_flush:
                flush.fill_(i & 0xFF)  # outside the events
            ev[i][0].record(stream)
            run()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in ev]

    warm = event_pass(False)
    cold = event_pass(True)

    # each launch of the step on its own, eagerly, with events between them
    # routing is two launches (scores, then the top-k selection), timed apart
    names = ["encode_kernel"] + (["route_kernel", "select_kernel"] if wl.routed else []) + ["attn_kernel"]
    if not fused and wl.value_basis != "identity":
        names.append("upproject_kernel")
    per = {n: 0.0 for n in names}
    evs = []
    for _ in range(steps):  # enqueued back to back: the host runs ahead of the GPU
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        evs.append(ev)
        ev[0].record(stream)
        i = 0
        sess.prepare()
        i += 1
        ev[i].record(stream)
        if wl.routed:
            sess.score()
            i += 1
            ev[i].record(stream)
            sess.select()
            i += 1
            ev[i].record(stream)
        if fused and wl.value_basis != "identity":
            sess.attend_upproject()
        else:
            sess.attend()
        i += 1
        ev[i].record(stream)
        if not fused and wl.value_basis != "identity":
            sess.upproject()
            i += 1
            ev[i].record(stream)
    torch.cuda.synchronize()
    for ev in evs:
        for k, n in enumerate(names):
            per[n] += ev[k].elapsed_time(ev[k + 1]) * 1e3
    kb = step_bytes(sess)
    kernels = {}
    for n in names:
        us = per[n] / steps
        rec = {"avg_us": round(us, 2)}
        if n in kb:
            gbps = kb[n] / (us * 1e-6) / 1e9
            rec.update(algo_bytes=kb[n], achieved_gbps=round(gbps, 1),
                       frac=round(gbps / HBM_PEAK_GBPS, 4))
        cnt = measured_counters(n, wl.name)
        rec.update(cnt if cnt else {"mfma_busy_pct": None, "valu_busy_pct": None})
        kernels[n] = rec
    if g is not None:
        # leave the buffers as a replay of the step leaves them
        g.replay()
        torch.cuda.synchronize()
        del g

    total = sum(kb.values())
    ms = wall_s * 1e3 / steps
    dom = "route_kernel" if wl.routed else "attn_kernel"
    dom_us = kernels[dom]["avg_us"]
    ach = kb[dom] / (dom_us * 1e-6) / 1e9
    return {
        "wall_s": wall_s, "ms_per_step": ms, "kv_tokens": sess.kv_tokens(),
        "value": sess.kv_tokens() * steps / wall_s,
        "step_algo_bytes": total,
        "step_hbm_frac": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "step_time_us": {"warm": spread(warm), "cold_after_1GiB_fill": spread(cold)},
        "step_hbm_frac_median": {
            "warm": round(total / (pct(warm, 50) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "cold_after_1GiB_fill": round(total / (pct(cold, 50) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)},
        "kernels": kernels,
        "roofline": {
            "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(dom, wl.name),
            "kernel": dom, "algo_bytes_per_launch": kb[dom], "avg_launch_us": dom_us},
    }


def config_of(sess) -> dict:
    wl = sess.wl
    return {
        "workload": wl.name, "batch": wl.batch, "context": (sum(sess.seq_lens) // wl.batch),
        "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
        "page_size": wl.page_size, "rank_v": wl.rank_v, "rank_k": wl.rank_k,
        "storage": wl.storage, "latents": wl.lat_storage, "keys": wl.key_mode,
        "topk": f"{wl.topk_num}/{wl.topk_den}" if wl.routed else "all",
        "append_per_seq": wl.append_per_seq, "parallelism": "single-gpu",
    }


def planted_recall(sess):
    """Share of the planted pages that routing chose (70B share workload)."""
    wl = sess.wl
    if not (wl.routed and wl.planted_frac > 0):
        return None
    sel = sess.sel.cpu()
    got = tot = 0
    for b in range(wl.batch):
        N = -(-sess.seq_lens[b] // wl.page_size)
        planted = set(synth.planted_pages(wl, b, N).tolist())
        for g in range(wl.num_kv_heads):
            chosen = set(sel[b, g].tolist())
            got += len(planted & chosen)
            tot += len(planted)
    return round(got / tot, 4) if tot else None


def sub_record(name, args, flush) -> dict:
    wl = WORKLOADS[name]
    log(f"[bench] staging workload {wl.name}")
    sess = DecodeSession(wl, "cuda")
    torch.cuda.synchronize()
    m = measure(sess, args.sub_steps, args.warmup, not args.eager, args.fused, flush)
    rec = {"config": config_of(sess), "value": round(m["value"], 1), "unit": "KV-tokens/s",
           "ms_per_step": round(m["ms_per_step"], 4)}
    rec.update({k: m[k] for k in ("step_algo_bytes", "step_hbm_frac", "step_time_us",
                                   "step_hbm_frac_median", "kernels", "roofline")})
    pr = planted_recall(sess)
    if pr is not None:
        rec["planted_recall"] = pr
    del sess
    torch.cuda.empty_cache()
    return rec


def copy_bandwidth(reps: int = 20) -> float:
    """Best plain device copy on this GPU (1 GiB to 1 GiB), GB/s moved."""
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        y.copy_(x)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3
        best = t if best is None else min(best, t)
    del x, y
    return 2 * n / best / 1e9


# ----------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, timed on the host; the same leg
# checks the timed step's page sets and outputs against the oracle
# ----------------------------------------------------------------------------

def cpu_baseline(sess, budget_s: float):
    """The oracle on whole (sequence, KV head) pairs until the time budget is
    spent; rate scaled to KV-tokens/s of the full step. Pairs of the first
    pass are also compared with the GPU's timed buffers (outside the timed
    oracle calls): page sets under the tie-band rule, z and o against the
    oracle evaluated on the GPU's accepted set, the new tokens' latents
    against the oracle's encode."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from tests import gpu_harness as H

    wl = sess.wl
    seqs = list(range(wl.batch))
    np.random.default_rng(0).shuffle(seqs)
    order = [(b, g) for b in seqs for g in range(wl.num_kv_heads)]
    memo = {}
    spent, tokens, pairs, passes = 0.0, 0, 0, 0
    cache, cached_bytes = [], 0
    par = {"pairs_checked": 0, "pairs_accepted": 0, "tie_band_pages": 0, "max_rel_err": 0.0,
           "encode_within_bound": 0}
    while spent < budget_s:
        passes += 1
        items = cache if passes > 1 else (_oracle_inputs(sess, b, g, memo) for b, g in order)
        for item in items:
            t0 = time.perf_counter()
            res = _oracle_pair(wl, sess.scale, item)
            spent += time.perf_counter() - t0
            tokens += item["L"]
            pairs += 1
            if passes == 1:
                _check_pair(sess, item, res, par, H)
            if passes == 1 and cached_bytes < CPU_CACHE_BYTES:
                cache.append(item)
                cached_bytes += sum(a.nbytes for a in item["prefix"].values())
            if spent >= budget_s:
                break
        if not cache:
            break
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    value = tokens / wl.num_kv_heads / spent
    n = par["pairs_checked"]
    parity = {
        "pairs_checked": n, "pairs_total": wl.batch * wl.num_kv_heads,
        "idx_parity": round(par["pairs_accepted"] / n, 6) if n else None,
        "tie_band_pages": par["tie_band_pages"],
        "max_rel_err": float(f"{par['max_rel_err']:.3e}"),
        "encode_within_bound": par["encode_within_bound"],
        "rule": "page sets bit-exact outside the band 1e-4*max(1,|s_k|) (+ the exact score shift "
                "of the new tokens' stored latents); z, o: max|gpu-ref|/||ref||_2 <= 5e-3",
    }
    base = {
        "value": value, "unit": "KV-tokens/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"{pairs} (sequence, KV head) pair runs, {passes} pass(es) over the "
                   f"{wl.batch * wl.num_kv_heads} pairs taken sequence by sequence in shuffled "
                   f"order (later passes repeat the first {len(cache)}), {tokens} context "
                   f"tokens, {spent:.1f} s of float64 numpy on the host; "
                   f"rate = tokens / H_kv / seconds"),
        "host_cpus": len(os.sched_getaffinity(0)),
    }
    return base, parity


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
        "b": b, "g": g, "prefix": prefix,
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
    res["o_up"] = O.upproject(res["z"], f["B_v"])
    res["state"] = st
    return res


def _check_pair(sess, it, res, par, H):
    import numpy as np

    import oracle as O

    wl = sess.wl
    b, g, L, P, G = it["b"], it["g"], it["L"], wl.page_size, wl.group
    par["pairs_checked"] += 1
    try:
        H.check_encode(sess, b, g)
        par["encode_within_bound"] += 1
    except AssertionError:
        pass
    if wl.routed:
        slack = H.new_token_slack(sess, b, g, res["state"])
        gsel = sess.sel[b, g].cpu().numpy()
        ok, band = H.accepted_selection(res["scores"], len(res["sel"]), gsel, slack)
        par["tie_band_pages"] += band
        if not ok:
            return
        pages = [int(j) for j in gsel if j >= 0]
    else:
        pages = list(range(-(-L // P)))
    par["pairs_accepted"] += 1
    if pages == list(res["sel"]):
        z, o = res["z"], res["o_up"]
    else:
        z, o, _ = O.attend_selected(it["q"], res["state"], it["f"], L, P, pages,
                                    key_mode=wl.key_mode, scale=sess.scale)
    zg = H.f64(sess.z[b, g * G:(g + 1) * G])
    og = H.f64(sess.o[b, g * G:(g + 1) * G])
    err = max(H.rel_err(zg, z), H.rel_err(og, o) if wl.value_basis != "identity" else 0.0)
    par["max_rel_err"] = max(par["max_rel_err"], float(np.float64(err)))


# ----------------------------------------------------------------------------

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
                         "traffic": measured_traffic("moments_mfma_kernel", wl.name),
                         "kernel": "moments_mfma_kernel", "kernel_algo_bytes": kernel_algo},
            "mfma_tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "fit_factors_call_ms": round(fit_ms, 2)}


def time_joint_fit(reps: int = 5):
    """The joint decoder fit on calibration samples at the 8B layer's shapes
    (32 query heads of 8 KV heads, every partition's latents at once):
    kvlr_fit_joint_moments timed with HIP events, and the whole synchronous
    kvlr_fit_joint call (moments, copy to host, float64 Cholesky solve over
    the 4096 output columns, fold into F = W_o D^T) by wall clock."""
    from decode_attention_rank_amd.fit import JointFit
    from decode_attention_rank_amd.workloads import DEFAULT_FIT_WORKLOAD, FIT_WORKLOADS

    wl = FIT_WORKLOADS[DEFAULT_FIT_WORKLOAD]
    n = JOINT_SAMPLES
    Hq, d, r = wl.num_q_heads, wl.head_dim, wl.rank_v
    x = synth.make_output_samples(wl, n, device="cuda")
    factors = synth.make_factors(wl, "cuda")
    from decode_attention_rank_amd import _lib as K
    kf = K.make_factors(**factors)
    hidden = synth.output_width(wl)
    W_o = synth.make_output_weight(wl, "cuda")
    jf = JointFit(wl, n, hidden)
    stream = torch.cuda.current_stream()
    jf.fit(kf, x, W_o)
    for _ in range(2):
        jf.moments(kf, x, n)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        jf.moments(kf, x, n)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    t0 = time.perf_counter()
    for _ in range(2):
        jf.fit(kf, x, W_o)
    call_ms = (time.perf_counter() - t0) * 1e3 / 2
    nl, nx = Hq * r, Hq * d
    flops = 2.0 * n * (Hq * d * r + nl * nl + nl * nx)   # Z = X A, Z^T Z, Z^T X
    del x
    return {"workload": wl.name, "samples": n, "num_q_heads": Hq, "latents": nl, "outputs": nx,
            "hidden": hidden,
            "timed": "kvlr_fit_joint_moments: latent outputs and the moments Z^T Z, Z^T X",
            "moments_call_us": round(us, 1), "mfma_f32_tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "fit_joint_call_ms": round(call_ms, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sub-steps", type=int, default=30, help="steps per other workload")
    ap.add_argument("--workload", default=DEFAULT_BENCH_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--others", default="configs",
                    help="other workloads to report: 'configs', 'all', 'none' or a comma list")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fit", action="store_true", help="skip the factor-fit measurement")
    ap.add_argument("--eager", action="store_true", help="launch the step's calls one by one "
                    "instead of replaying them as a HIP graph")
    ap.add_argument("--separate-upproject", action="store_true",
                    help="up-projection as its own launch instead of in attention's merge launch")
    args = ap.parse_args()
    args.fused = not args.separate_upproject

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    wl = WORKLOADS[args.workload]
    log(f"[bench] staging workload {wl.name}")
    t0 = time.time()
    sess = DecodeSession(wl, "cuda")
    torch.cuda.synchronize()
    log(f"[bench] staged in {time.time() - t0:.1f}s; KV tokens/step {sess.kv_tokens()}")
    m = measure(sess, args.steps, args.warmup, not args.eager, args.fused, flush)
    log(f"[bench] timed {args.steps} steps in {m['wall_s']:.3f}s")

    out = {
        "metric": METRIC, "value": round(m["value"], 1), "unit": "KV-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(m["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "config": config_of(sess),
        "launch": "eager" if args.eager else "hip-graph",
        "step_algo_bytes": m["step_algo_bytes"],
        "kernel_algo_bytes": step_bytes(sess),
        "step_hbm_frac": m["step_hbm_frac"],
        "step_time_us": m["step_time_us"],
        "step_hbm_frac_median": m["step_hbm_frac_median"],
        "kernels": m["kernels"],
        "roofline": m["roofline"],
    }
    pr = planted_recall(sess)
    if pr is not None:
        out["planted_recall"] = pr

    # the oracle leg runs on the headline workload's buffers as the timed
    # step left them, before anything else touches the GPU
    parity = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample (and checking the step against it)")
        out["cpu_baseline"], parity = cpu_baseline(sess, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    out["parity"] = parity

    if args.others == "none":
        others = []
    elif args.others == "configs":
        others = OTHER_WORKLOADS
    elif args.others == "all":
        others = OTHER_WORKLOADS + VARIANT_WORKLOADS
    else:
        others = [x for x in args.others.split(",") if x]
    others = [x for x in others if x != wl.name]
    if others:
        out["workloads"] = {}
        for name in others:
            out["workloads"][name] = sub_record(name, args, flush)
            log(f"[bench] {name}: {out['workloads'][name]['ms_per_step']} ms/step")

    out["copy_GBps"] = round(copy_bandwidth(), 1)
    if wl.storage == "bf16":
        out["output_projection"] = time_output_projection(sess)
    if not args.no_fit:
        log("[bench] timing the factor fit")
        out["factor_fit"] = time_factor_fit()
        log("[bench] timing the joint decoder fit")
        out["joint_fit"] = time_joint_fit()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
