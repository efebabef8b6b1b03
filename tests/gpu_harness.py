"""Shared checks for the GPU parity tests.

The oracle's inputs are rebuilt from the seeded generator (never read back
from what the HIP kernels wrote): the synthesized prefix rows plus the raw new
keys and values, which the oracle encodes itself.

Tolerances (derived in the design notes):
  * selected pages: bit-exact, except pages whose oracle score lies within
    tau = 1e-4 * max(1, |s_k|) of the k-th largest score s_k;
  * z, o: max_i |gpu - ref| / ||ref||_2 <= 5e-3 per (sequence, head), with the
    reference evaluated on the GPU's own accepted page set;
  * lse: absolute 2e-3 (natural log units);
  * encode: one unit in the last place of the stored type plus the float32
    accumulation bound n * 2**-24 * sum |a_i b_i| (see check_encode).
"""

from __future__ import annotations

import numpy as np
import torch

import oracle as O

OUT_TOL = 5e-3
LSE_TOL = 2e-3
TIE_REL = 1e-4


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def factors_np(sess, g: int) -> dict:
    """KV head g's factors; with per-head residual ranks only the kept
    residual coordinates (the GPU ignores the rest of A_k and B_k)."""
    f = {k: (None if v is None else f64(v[g])) for k, v in sess.factors.items()}
    r = sess.wl.k_rank(g)
    f["A_k"] = f["A_k"][:, :r]
    f["B_k"] = f["B_k"][:r]
    return f


def k_cols(sess, g: int, x: np.ndarray) -> np.ndarray:
    """The kept residual (or key-latent) coordinates of head g's rows."""
    return x[..., :sess.wl.k_rank(g)]


def oracle_state(sess, b: int, g: int) -> dict:
    """Oracle cache of (b, g) after the step's append: seeded prefix + oracle encode."""
    wl = sess.wl
    L0, n = sess.lens_before[b], sess.n_new[b]
    rows = sess.prefix_rows(b)
    st = {k: f64(v[g]) for k, v in rows.items()}
    st["k_lat"] = k_cols(sess, g, st["k_lat"])
    if n:
        off = sum(sess.n_new[:b])
        Kn = f64(sess.k_new[off:off + n, g])
        Vn = f64(sess.v_new[off:off + n, g])
        f = factors_np(sess, g)
        st = O.append_tokens(st, L0, Kn, Vn, f["A_v"], f["A_k"], f["W_pred"],
                             key_mode=wl.key_mode, storage=wl.lat_storage)
    return st


def oracle_states(sess, b: int) -> list:
    """oracle_state of every KV head of sequence b (one draw of the prefix)."""
    wl = sess.wl
    L0, n = sess.lens_before[b], sess.n_new[b]
    rows = sess.prefix_rows(b)
    out = []
    for g in range(wl.num_kv_heads):
        st = {k: f64(v[g]) for k, v in rows.items()}
        st["k_lat"] = k_cols(sess, g, st["k_lat"])
        if n:
            off = sum(sess.n_new[:b])
            Kn = f64(sess.k_new[off:off + n, g])
            Vn = f64(sess.v_new[off:off + n, g])
            f = factors_np(sess, g)
            st = O.append_tokens(st, L0, Kn, Vn, f["A_v"], f["A_k"], f["W_pred"],
                                 key_mode=wl.key_mode, storage=wl.lat_storage)
        out.append(st)
    return out


def pages_kept(sess, b: int, N: int) -> int:
    """k_b of sequence b: its budget when the session routes with per-sequence
    budgets (capped by the page count), else the workload's fraction."""
    if getattr(sess, "k_pages_cpu", None) is not None:
        return min(N, max(sess.k_pages_cpu[b], 0)) if N > 0 else 0
    return O.pages_to_keep(N, sess.wl.topk_num, sess.wl.topk_den)


def check_selection(sess, b: int, g: int, st: dict, slack: float = 0.0,
                    gpu_sel=None, gpu_scores=None) -> int:
    """The GPU's page set and page scores of (b, g) against the oracle's
    scores of the same cache; returns the number of pages in the tie band."""
    wl = sess.wl
    P, L = wl.page_size, sess.seq_lens[b]
    f = factors_np(sess, g)
    N = -(-L // P)
    S = O.page_scores(q_group(sess, b, g), st["v"], st["k_lat"], f["W_pred"], f["B_k"], L, P)
    k = pages_kept(sess, b, N)
    gsel = sess.sel[b, g].cpu().numpy() if gpu_sel is None else gpu_sel
    ok, band = accepted_selection(S, k, gsel, slack)
    assert ok, f"pair ({b},{g}): GPU pages {sorted(gsel[gsel >= 0].tolist())[:16]}... not accepted"
    if N:
        gs = f64(sess.page_scores[b, g, :N]) if gpu_scores is None else gpu_scores[:N]
        tol = TIE_REL * np.maximum(1.0, np.abs(S)) + slack
        assert np.all(np.abs(gs - S) <= tol), f"pair ({b},{g}): page scores off by {np.abs(gs - S).max()}"
    return band


def q_group(sess, b: int, g: int) -> np.ndarray:
    G = sess.wl.group
    return f64(sess.q[b, g * G:(g + 1) * G])


def accepted_selection(S: np.ndarray, k: int, gpu_sel, slack: float = 0.0) -> tuple[bool, int]:
    """Tie-band acceptance of a GPU page set; returns (ok, pages inside the band)."""
    gset = [int(j) for j in gpu_sel if j >= 0]
    if k == 0:
        return len(gset) == 0, 0
    if len(gset) != k or len(set(gset)) != k or gset != sorted(gset):
        return False, 0
    sk = np.sort(S)[::-1][k - 1]
    tau = TIE_REL * max(1.0, abs(sk)) + slack
    must = set(np.nonzero(S > sk + tau)[0].tolist())
    may = set(np.nonzero(S >= sk - tau)[0].tolist())
    G = set(gset)
    band = len(may - must)
    return must <= G and G <= may, band


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max_i |gpu - ref| / ||ref||_2 over the last axis, worst row."""
    gpu = np.atleast_2d(gpu)
    ref = np.atleast_2d(ref)
    num = np.abs(gpu - ref).max(axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    out = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    return float(out.max()) if out.size else 0.0


def stage_oracle_sequence(sess, b: int) -> list:
    """Overwrite sequence b's pages with the oracle's own cache (all KV heads),
    so a following GPU decode reads exactly the oracle's stored values.
    Returns the per-head oracle states."""
    states = [oracle_state(sess, b, g) for g in range(sess.wl.num_kv_heads)]
    L = sess.seq_lens[b]

    def head_rows(st, k):
        x = st[k][:L]
        if k == "k_lat":  # per-head residual ranks: pad to the full width
            x = np.pad(x, ((0, 0), (0, sess.wl.rank_k - x.shape[1])))
        return x
    rows = {k: torch.from_numpy(np.stack([head_rows(st, k) for st in states])) for k in states[0]}
    sess.write_rows(b, rows)
    return states


def new_token_slack(sess, b: int, g: int, st: dict) -> float:
    """How far a routing score can move because the GPU's stored latents of
    the new tokens differ from the oracle's (check_encode bounds each
    difference by one unit in the last place of the stored type plus the
    float32 accumulation error): with the actual differences dv, dc,
    sum_i |q_hat_i| |dv_i| + sum_i |q_tilde_i| |dc_i|, worst token and head."""
    wl = sess.wl
    n = sess.n_new[b]
    if not wl.routed or n == 0:
        return 0.0
    f = factors_np(sess, g)
    qh, qt = O.project_queries(q_group(sess, b, g), f["W_pred"], f["B_k"])
    L0 = sess.lens_before[b]
    got = {k: f64(v[g]) for k, v in sess.read_rows(b, L0 + n, L0).items()}
    got["k_lat"] = k_cols(sess, g, got["k_lat"])
    dv = np.abs(got["v"] - st["v"][L0:L0 + n])
    dc = np.abs(got["k_lat"] - st["k_lat"][L0:L0 + n])
    bound = np.abs(qh) @ dv.T + np.abs(qt) @ dc.T   # [G, n]
    return float(bound.max()) * 1.01 + 1e-6


def check_pair(sess, b: int, g: int, *, state=None, check_scores=True, slack=0.0) -> dict:
    """Compare the GPU step's outputs for (b, g) against the oracle. `slack`
    widens the page-score tolerance and the tie band (end-to-end runs, where
    the GPU encoded the new tokens itself)."""
    wl = sess.wl
    G, P, L = wl.group, wl.page_size, sess.seq_lens[b]
    st = oracle_state(sess, b, g) if state is None else state
    f = factors_np(sess, g)
    q = q_group(sess, b, g)
    info = {}
    if wl.routed:
        N = -(-L // P)
        S = O.page_scores(q, st["v"], st["k_lat"], f["W_pred"], f["B_k"], L, P)
        k = pages_kept(sess, b, N)
        gsel = sess.sel[b, g].cpu().numpy()
        ok, band = accepted_selection(S, k, gsel, slack)
        assert ok, f"pair ({b},{g}): GPU pages {sorted(gsel[gsel >= 0].tolist())[:16]}... not accepted"
        info["tie_band"] = band
        pages = [int(j) for j in gsel if j >= 0]
        if getattr(sess, "sel_phys", None) is not None:
            # the physical pages written beside the ids: page-table entries, -1 padding
            gphys = sess.sel_phys[b, g].cpu().numpy()
            want = np.full(len(gsel), -1, np.int64)
            want[:len(pages)] = sess.page_table_cpu[b][pages].numpy()
            assert np.array_equal(gphys, want), f"pair ({b},{g}): physical pages differ from the table"
        if check_scores and N:
            gs = f64(sess.page_scores[b, g, :N])
            tol = TIE_REL * np.maximum(1.0, np.abs(S)) + slack
            assert np.all(np.abs(gs - S) <= tol), f"page scores off by {np.abs(gs - S).max()}"
            assert np.all(np.isneginf(f64(sess.page_scores[b, g, N:])))
    else:
        pages = list(range(-(-L // P)))
    z, o, lse = O.attend_selected(q, st, f, L, P, pages, key_mode=wl.key_mode, scale=sess.scale)
    zg = f64(sess.z[b, g * G:(g + 1) * G])
    og = f64(sess.o[b, g * G:(g + 1) * G])
    lg = f64(sess.lse[b, g * G:(g + 1) * G])
    info["z_err"] = rel_err(zg, z)
    info["o_err"] = rel_err(og, o)
    assert info["z_err"] <= OUT_TOL, f"z rel err {info['z_err']}"
    assert info["o_err"] <= OUT_TOL, f"o rel err {info['o_err']}"
    if np.all(np.isinf(lse)):
        assert np.all(np.isneginf(lg))
    else:
        info["lse_err"] = float(np.abs(lg - lse).max())
        assert info["lse_err"] <= LSE_TOL, f"lse err {info['lse_err']}"
    return info


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |x| (normal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    _, e = np.frexp(ax)
    return np.ldexp(1.0, e - 8)


def fp8_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of OCP E4M3 values at |x| (2**-9 in the subnormal range)."""
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e - 4, -9))


def check_encode(sess, b: int, g: int) -> dict:
    """GPU-written latents of (b, g)'s new tokens against the oracle's encode.

    The kernel accumulates in float32 and then rounds once to the storage
    type, so an element may differ from the oracle's correctly rounded value
    by one unit in the last place of the stored type plus the float32
    accumulation error, bounded by gamma * sum_i |a_i b_i| with
    gamma = n * 2**-24 for n accumulated terms. The residual latent also
    inherits the GPU's own stored value latent, through |dv| |W_pred A_k|.
    """
    wl = sess.wl
    L0, n = sess.lens_before[b], sess.n_new[b]
    if n == 0:
        return {}
    off = sum(sess.n_new[:b])
    f = factors_np(sess, g)
    Kn = f64(sess.k_new[off:off + n, g])
    Vn = f64(sess.v_new[off:off + n, g])
    enc = O.encode_tokens(Kn, Vn, f["A_v"], f["A_k"], f["W_pred"], key_mode=wl.key_mode,
                          storage=wl.lat_storage)
    got = {k: f64(v[g]) for k, v in sess.read_rows(b, L0 + n, L0).items()}
    got["k_lat"] = k_cols(sess, g, got["k_lat"])
    d, rv = wl.head_dim, wl.rank_v
    u = 2.0 ** -24
    if wl.lat_storage == "fp8":
        def unit(x, y):
            return fp8_ulp(np.maximum(np.abs(x), np.abs(y)))
    elif wl.lat_storage == "bf16":
        def unit(x, y):
            return bf16_ulp(np.maximum(np.abs(x), np.abs(y)))
    else:
        def unit(x, y):
            return np.maximum(np.abs(x), np.abs(y)) * 2.0 ** -23
    info = {}
    # value latent: d products per element
    tol_v = unit(enc["v"], got["v"]) + d * u * (np.abs(Vn) @ np.abs(f["A_v"]))
    dv = np.abs(got["v"] - enc["v"])
    assert np.all(dv <= tol_v), f"v off by {(dv / tol_v).max():.2f} x tolerance"
    info["v_frac_off"] = float((dv > 0).mean())
    if wl.key_mode == "exact":
        M = f["W_pred"] @ f["A_k"]
        absM = np.abs(M)
        terms = np.abs(Kn) @ np.abs(f["A_k"]) + np.abs(got["v"]) @ absM
        m_err = d * u * (np.abs(f["W_pred"]) @ np.abs(f["A_k"])) + 2.0 ** -16 * absM
        tol_c = (unit(enc["k_lat"], got["k_lat"]) + (d + 2 * rv) * u * terms
                 + dv @ absM + np.abs(got["v"]) @ m_err)
    else:
        tol_c = unit(enc["k_lat"], got["k_lat"]) + d * u * (np.abs(Kn) @ np.abs(f["A_k"]))
    dc = np.abs(got["k_lat"] - enc["k_lat"])
    assert np.all(dc <= tol_c), f"k_lat off by {(dc / tol_c).max():.2f} x tolerance"
    info["k_lat_frac_off"] = float((dc > 0).mean())
    if wl.key_mode == "exact":
        assert np.array_equal(got["k_exact"], enc["k_exact"]), "original keys not copied exactly"
    return info
