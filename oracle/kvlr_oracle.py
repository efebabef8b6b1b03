"""Oracle: one decode step of attention read from a low-rank compressed, paged
KV cache, in the BasisKV form, written as plainly as possible in float64.

TEST INFRASTRUCTURE ONLY. Callers: the test suite, the smoke check and the
CPU-baseline leg of the benchmark. Nothing in the HIP library or its binding
imports this file, and this file imports nothing from them. It shares no
kernels, helpers, tables or constants with the GPU path.

Source: "BasisKV: Value Latents for Communication and Key Routing".
  * English abstract: K and V are compressed by low-rank projections; the
    value cache keeps rank-r_v latents; the stored V latent is reused to
    predict part of each key for page routing, and a key-specific residual
    holds what the V latent cannot recover; original keys are then fetched only
    for the chosen pages, where exact QK scores are computed; value
    compression is tied to the output projection.
  * Method-details section: a low-rank cache compression module plus a
    key-routing prediction module that predicts part of the key information.
  * Key-points section: the shared low-rank value representation narrows the
    value cache.

Everything is computed in the plain, decompressed form: keys and values are
expanded back to head_dim before any dot product with the query. The GPU path
works in latent space instead (an exact reassociation), so the two agree only
up to rounding, never by sharing an evaluation order.

Readings taken where the page leaves a step open (each is listed again in the
design notes):
  R1  the key prediction is linear: K_pred = v . W_pred, W_pred of shape
      [r_v, d] per KV head;
  R2  the residual is taken against the STORED (rounded) V latent, the only
      one available when routing;
  R3  the residual is encoded by a rank-r_k projection c = (K - K_pred) . A_k
      and decoded by c . B_k;
  R4  a page's routing score is the max over its valid tokens and over the
      query heads of its KV group of the unscaled approximate score q . K~;
  R5  ties between equal page scores go to the lower logical page index; the
      chosen pages are returned in ascending order;
  R6  k_b = min(N_b, max(1, ceil(N_b * num / den))) pages per (sequence,
      KV head); k_b = 0 when N_b = 0;
  R7  no forced pages (no sink or recent window): pure top-k;
  R8  tokens at positions >= L_b are ignored in routing and attention;
  R9  scores use scale = 1/sqrt(head_dim) unless the caller passes another;
  R10 in routed mode the softmax runs over the selected tokens only;
  R11 the up-projection B_v is applied once per query head to z = sum p v;
  R12 in dense ("latent keys") mode scores use the decompressed latent key
      k . B_k and every page is attended;
  R13 an empty context (L_b = 0) gives z = 0, o = 0 and lse = -inf.

Storage: latents are rounded to the storage type ("bf16", "f32", "fp8" for
OCP E4M3 saturating at +-448, or "f64" for no rounding) with
round-to-nearest-even; every input value (keys, values, factors, queries) is
taken exactly as given.
"""

from __future__ import annotations

import math

import numpy as np

STORAGE_TYPES = ("bf16", "f32", "fp8", "f64")

# Largest finite bfloat16: significand 1.1111111b, exponent 127.
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


# ----------------------------------------------------------------------------
# Storage rounding
# ----------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even; result as float64.

    bfloat16 keeps the float32 exponent range and an 8-bit significand
    (1 implicit + 7 stored bits), so for |x| in [2**(e-1), 2**e) the spacing
    of representable values is 2**(e-8); below the smallest normal 2**-126 the
    spacing stays 2**-133 (subnormals). np.rint rounds halves to even.
    Pinned against torch's float32 -> bfloat16 conversion (a library RNE).
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)
    spacing = np.ldexp(1.0, np.maximum(e - 8, -133))
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.rint(ax / spacing) * spacing
        r = np.where(r > _BF16_MAX, np.inf, r)
        out = np.copysign(r, x)
    return np.where(np.isfinite(x), out, x)


# Largest finite OCP 8-bit E4M3 value: significand 1.110b, exponent 8 (the
# all-ones pattern is NaN; the format has no infinities).
_FP8_E4M3_MAX = 448.0


def round_fp8_e4m3(x) -> np.ndarray:
    """Round to the nearest OCP 8-bit floating point E4M3 value, ties to even,
    saturating at +-448; NaN stays NaN (infinities saturate). Result as
    float64.

    E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 stored significand bits.
    For |x| in [2**(e-1), 2**e) the spacing is 2**(e-4); normal values start
    at 2**-6 and below that the spacing stays 2**-9 (subnormals). The latent
    codec of the FP8 variant (a lossy latent store in the spirit of the page
    "PackKV: Reducing KV Cache Memory Footprint through LLM-Aware Lossy
    Compression", abstract) rounds each latent once with this function.
    Pinned against torch's float32 -> float8_e4m3fn conversion inside the
    range, the format's printed extreme values, and tie cases.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)
    spacing = np.ldexp(1.0, np.maximum(e - 4, -9))
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.minimum(np.rint(ax / spacing) * spacing, _FP8_E4M3_MAX)
        r = np.where(np.isinf(ax), _FP8_E4M3_MAX, r)
        out = np.copysign(r, x)
    return np.where(np.isnan(x), x, out)


def round_to_storage(x, storage: str) -> np.ndarray:
    """Value that the cache holds after storing x in the given type."""
    x = np.asarray(x, dtype=np.float64)
    if storage == "f64":
        return x.copy()
    if storage == "f32":
        return x.astype(np.float32).astype(np.float64)
    if storage == "bf16":
        return round_bf16(x)
    if storage == "fp8":
        return round_fp8_e4m3(x)
    raise ValueError(f"unknown storage type {storage!r}")


# ----------------------------------------------------------------------------
# Append-side encode (BasisKV English abstract: low-rank K/V projections;
# V latent reused to predict part of the key; key-specific residual)
# ----------------------------------------------------------------------------

def encode_tokens(K, V, A_v, A_k, W_pred=None, *, key_mode: str, storage: str):
    """Encode new tokens of one KV head.

    K, V: [n, d] values of the new keys and values. A_v: [d, r_v]. A_k: [d, r_k].
    key_mode "exact" (routed BasisKV): v = store(V A_v);
        c = store((K - v W_pred) A_k) with v the stored latent (R2, R3);
        the original key is kept as given.
    key_mode "latent" (dense low-rank keys): v = store(V A_v); k = store(K A_k).
    Returns dict with "v", "k_lat" (residual c or key latent k) and, in exact
    mode, "k_exact".
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    v = round_to_storage(V @ np.asarray(A_v, np.float64), storage)
    if key_mode == "exact":
        if W_pred is None:
            raise ValueError("exact-key mode needs W_pred")
        K_pred = v @ np.asarray(W_pred, np.float64)
        c = round_to_storage((K - K_pred) @ np.asarray(A_k, np.float64), storage)
        return {"v": v, "k_lat": c, "k_exact": K.copy()}
    if key_mode == "latent":
        k = round_to_storage(K @ np.asarray(A_k, np.float64), storage)
        return {"v": v, "k_lat": k}
    raise ValueError(f"unknown key mode {key_mode!r}")


def empty_state(capacity: int, d: int, r_v: int, r_k: int, key_mode: str):
    """Logical cache of one (sequence, KV head): row t holds token t."""
    st = {
        "v": np.zeros((capacity, r_v)),
        "k_lat": np.zeros((capacity, r_k)),
    }
    if key_mode == "exact":
        st["k_exact"] = np.zeros((capacity, d))
    return st


def append_tokens(state, L_before: int, K_new, V_new, A_v, A_k, W_pred=None, *,
                  key_mode: str, storage: str):
    """Write the encoded new tokens at logical positions L_before, L_before+1, ...

    Paging only decides where a token lands physically: token position p sits
    in logical page p // P at slot p % P. The oracle keeps the logical order.
    """
    enc = encode_tokens(K_new, V_new, A_v, A_k, W_pred, key_mode=key_mode, storage=storage)
    n = enc["v"].shape[0]
    out = {name: arr.copy() for name, arr in state.items()}
    need = L_before + n
    for name in out:
        if out[name].shape[0] < need:
            grown = np.zeros((need, out[name].shape[1]))
            grown[: out[name].shape[0]] = out[name]
            out[name] = grown
    for name, rows in enc.items():
        out[name][L_before:need] = rows
    return out


# ----------------------------------------------------------------------------
# Query side and routing (BasisKV English abstract: the V latent predicts part
# of the key needed for routing; the key-specific residual adds the rest; the
# result decides which key pages are read)
# ----------------------------------------------------------------------------

def project_queries(q_group, W_pred, B_k):
    """Query images in latent space: q_hat = q W_pred^T, q_tilde = q B_k^T.

    These are what a latent-space scorer dots with the stored latents; the
    oracle's own routing does not use them (it decompresses instead).
    """
    q = np.asarray(q_group, np.float64)
    q_hat = None if W_pred is None else q @ np.asarray(W_pred, np.float64).T
    q_tilde = q @ np.asarray(B_k, np.float64).T
    return q_hat, q_tilde


def key_approximation(v, c, W_pred, B_k):
    """K~ = v W_pred + c B_k: predicted key part plus decoded residual (R1, R3)."""
    return np.asarray(v, np.float64) @ np.asarray(W_pred, np.float64) + \
        np.asarray(c, np.float64) @ np.asarray(B_k, np.float64)


def page_scores(q_group, v, c, W_pred, B_k, L: int, P: int):
    """Approximate routing score of each logical page of one (sequence, KV head).

    s[h, t] = q_h . K~_t over the valid tokens t < L; page j's score is the max
    of s over its valid tokens and over the heads of the group (R4, R8).
    Returns float64 array of length N = ceil(L / P).
    """
    N = -(-L // P)
    if N == 0:
        return np.zeros(0)
    Kt = key_approximation(np.asarray(v)[:L], np.asarray(c)[:L], W_pred, B_k)
    s = np.asarray(q_group, np.float64) @ Kt.T
    S = np.empty(N)
    for j in range(N):
        S[j] = s[:, j * P: min((j + 1) * P, L)].max()
    return S


def pages_to_keep(N: int, num: int, den: int) -> int:
    """k_b = min(N, max(1, ceil(N * num / den))), 0 for an empty sequence (R6)."""
    if N <= 0:
        return 0
    return min(N, max(1, -(-(N * num) // den)))


def select_top_pages(S, k: int):
    """The k pages with the largest scores; equal scores favour the lower page
    index (R5). Returned in ascending page order."""
    order = sorted(range(len(S)), key=lambda j: (-float(S[j]), j))
    return sorted(order[:k])


def tokens_of_pages(pages, L: int, P: int):
    """Valid token positions of the given logical pages, page by page."""
    out = []
    for j in pages:
        out.extend(range(j * P, min((j + 1) * P, L)))
    return np.asarray(out, dtype=np.int64)


# ----------------------------------------------------------------------------
# Attention and the up-projection (BasisKV English abstract: exact QK on the
# original keys of the chosen pages; value compression tied to the output
# projection)
# ----------------------------------------------------------------------------

def attend(q_group, keys, v_rows, B_v, scale: float):
    """Textbook softmax attention of the group's queries over the given tokens.

    keys: [T, d] (original keys, or decompressed latent keys); v_rows: [T, r_v]
    stored V latents. Values are decompressed as V^ = v B_v. Returns
    z = p v (latent output), o = p V^ (decompressed output) and
    lse = log(sum exp(scale q.k)) per head (natural log, scaled-score units).
    """
    q = np.asarray(q_group, np.float64)
    G = q.shape[0]
    r_v = np.asarray(B_v).shape[0]
    d_out = np.asarray(B_v).shape[1]
    keys = np.asarray(keys, np.float64)
    v_rows = np.asarray(v_rows, np.float64)
    if keys.shape[0] == 0:  # R13
        return np.zeros((G, r_v)), np.zeros((G, d_out)), np.full(G, -np.inf)
    s = scale * (q @ keys.T)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    w = p / l
    z = w @ v_rows
    V_hat = v_rows @ np.asarray(B_v, np.float64)
    o = w @ V_hat
    lse = (m + np.log(l))[:, 0]
    return z, o, lse


def upproject(z, B_v):
    """o = z B_v: one up-projection per query head (R11)."""
    return np.asarray(z, np.float64) @ np.asarray(B_v, np.float64)


def attend_selected(q_group, state, factors, L: int, P: int, pages, *,
                    key_mode: str, scale: float):
    """Attention of one (sequence, KV head) over the given logical pages."""
    t = tokens_of_pages(pages, L, P)
    if key_mode == "exact":
        keys = state["k_exact"][t]
    else:
        keys = np.asarray(state["k_lat"], np.float64)[t] @ np.asarray(factors["B_k"], np.float64)
    return attend(q_group, keys, state["v"][t], factors["B_v"], scale)


def decode_pair(q_group, state, factors, L: int, P: int, *, key_mode: str,
                scale: float | None = None, topk: tuple[int, int] | None = None):
    """One decode step for one (sequence, KV head).

    q_group: [G, d] queries of the heads sharing this KV head.
    state: logical cache rows ("v", "k_lat", "k_exact" in exact mode).
    factors: dict with "B_v", "B_k", and in exact mode "W_pred".
    Routed (exact) mode: score pages, keep the top k_b (R4-R7), attend with the
    original keys of those pages (R10). Latent mode: attend every page with the
    decompressed latent keys (R12).
    Returns dict(sel, scores, z, o, lse).
    """
    q = np.asarray(q_group, np.float64)
    d = q.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)  # R9
    N = -(-L // P)
    if key_mode == "exact":
        S = page_scores(q, state["v"], state["k_lat"], factors["W_pred"], factors["B_k"], L, P)
        num, den = topk if topk is not None else (1, 1)
        sel = select_top_pages(S, pages_to_keep(N, num, den))
    elif key_mode == "latent":
        S = None
        sel = list(range(N))
    else:
        raise ValueError(f"unknown key mode {key_mode!r}")
    z, o, lse = attend_selected(q, state, factors, L, P, sel, key_mode=key_mode, scale=scale)
    return {"sel": sel, "scores": S, "z": z, "o": o, "lse": lse}


# ----------------------------------------------------------------------------
# Output projection (BasisKV English abstract and method details, key
# innovation: the value latent is tied to the output projection, so one
# low-rank value representation narrows both the value cache and what the
# attention output carries)
# ----------------------------------------------------------------------------

def output_projection(o, W_o):
    """Plain attention output through the output projection.

    o: [n_heads, d] per-head outputs of one sequence (o_h = z_h B_v[g(h)]).
    W_o: [hidden, n_heads * d], rows are output features (the usual
    "out x in" layout). Returns [hidden] = W_o . concat_h(o_h).
    """
    o = np.asarray(o, np.float64).reshape(-1)
    return np.asarray(W_o, np.float64) @ o


def fold_output_weights(B_v_heads, W_o):
    """F = W_o . blockdiag(B_v^T): the output projection seen from the latents.

    B_v_heads: [n_heads, r_v, d], the up-projection of each query head's KV
    head. W_o: [hidden, n_heads * d]. Returns F [hidden, n_heads * r_v] with
    F[:, h r_v + e] = sum_j W_o[:, h d + j] B_v[h][e, j], so that
    F . concat_h(z_h) = W_o . concat_h(z_h B_v[h]) for every z.
    """
    B = np.asarray(B_v_heads, np.float64)
    W = np.asarray(W_o, np.float64)
    n_heads, r_v, d = B.shape
    cols = []
    for h in range(n_heads):
        W_h = W[:, h * d:(h + 1) * d]          # [hidden, d]
        cols.append(W_h @ B[h].T)             # [hidden, r_v]
    return np.concatenate(cols, axis=1)


def latent_output_projection(z, F):
    """[hidden] = F . concat_h(z_h) for one sequence (z: [n_heads, r_v])."""
    return np.asarray(F, np.float64) @ np.asarray(z, np.float64).reshape(-1)


# ----------------------------------------------------------------------------
# Factor fitting from sample keys and values of one KV head (BasisKV English
# abstract: low-rank K/V projections; the value latent predicts part of the
# key, a key-specific residual holds the rest; method details, key design).
# The pages do not give the fitting procedure; this is the plainest staged
# reading: principal directions of the values, least-squares prediction of
# the keys from the value latents, principal directions of what is left.
# ----------------------------------------------------------------------------

def _top_eigvecs(C, r):
    """Eigenvectors of the symmetric C for its r largest eigenvalues, largest
    first; each column's entry of largest magnitude made positive."""
    w, U = np.linalg.eigh(np.asarray(C, np.float64))
    order = np.argsort(w)[::-1][:r]
    w, U = w[order], U[:, order]
    for i in range(r):
        j = np.argmax(np.abs(U[:, i]))
        if U[j, i] < 0:
            U[:, i] = -U[:, i]
    return w, U


def fit_factors(K, V, r_v: int, r_k: int, *, key_mode: str):
    """Factors of one KV head from n sample keys and values ([n, d] each).

    A_v: top-r_v eigenvectors of V^T V; B_v = A_v^T.
    exact (routed) keys: W_pred = argmin_W |K - v W|^2 with v = V A_v, i.e.
      (v^T v)^-1 v^T K; A_k: top-r_k eigenvectors of R^T R, R = K - v W_pred.
    latent keys: A_k: top-r_k eigenvectors of K^T K; no W_pred.
    B_k = A_k^T. Returns dict of float64 arrays and the eigenvalues.
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    lam_v, A_v = _top_eigvecs(V.T @ V, r_v)
    out = {"A_v": A_v, "B_v": A_v.T.copy(), "lam_v": lam_v}
    if key_mode == "exact":
        v = V @ A_v
        W = np.linalg.solve(v.T @ v, v.T @ K)
        R = K - v @ W
        lam_k, A_k = _top_eigvecs(R.T @ R, r_k)
        out["W_pred"] = W
    else:
        lam_k, A_k = _top_eigvecs(K.T @ K, r_k)
        out["W_pred"] = None
    out.update(A_k=A_k, B_k=A_k.T.copy(), lam_k=lam_k)
    return out


def choose_residual_ranks(lam_k, energy_frac: float, allowed=(16, 32, 64)):
    """Per-head residual ranks for an adaptive residual (BasisKV method
    details, key design: a residual mechanism that adapts to what the value
    cannot recover; read here as a rank per KV head). lam_k: [H, r_max]
    residual eigenvalues, largest first. Head g gets the smallest allowed
    r <= r_max whose top-r eigenvalues hold at least energy_frac of the
    energy of all r_max (negative eigenvalues count as zero), else r_max."""
    lam = np.maximum(np.asarray(lam_k, np.float64), 0.0)
    H, r_max = lam.shape
    out = []
    for g in range(H):
        total = lam[g].sum()
        pick = r_max
        for r in allowed:
            if r <= r_max and lam[g, :r].sum() >= energy_frac * total:
                pick = r
                break
        out.append(pick)
    return out


# ----------------------------------------------------------------------------
# Joint fit of the value decoders across per-GPU attention partitions
# (BasisKV English abstract: the low-rank factors are optimised jointly across
# the per-GPU attention partitions against the complete attention output,
# not partition by partition; method details, key design: the loss couples
# every GPU's attention partition; key innovation: value compression is tied
# to the output projection). Reading taken here: the value encoders A_g stay
# as fitted (the cache's latents v = V A_g exist before any query), and the
# decoders that map latent outputs back to attention outputs are what the
# joint loss chooses. Head h's latent output is z_h = x_h A_g (x_h its exact
# attention output, sum_t p_t V_t, since z_h = sum_t p_t v_t); the complete
# output of a layer is y = W_o concat_h(x_h), reproduced as F concat_h(z_h)
# with the folded decoder F = W_o D^T.
#   staged:    D = blockdiag_h(A_g^T)          (B_v = A_v^T, head by head)
#   isolated:  partition p fits its own heads' outputs from its own latents
#   joint:     D = argmin sum_n |x_n - z_n D|^2 over all partitions at once
# For any W_o, argmin_F sum_n |W_o x_n - F z_n|^2 = W_o D_joint^T: the
# least-squares residual of D_joint is orthogonal to every latent, so one
# decoder serves every output projection.
# ----------------------------------------------------------------------------

def latent_outputs(X, A_heads, group: int):
    """z_h = x_h A_{h // group} for every query head h of every sample.

    X: [n, H_q, d] exact attention outputs; A_heads: [H_kv, d, r].
    Returns Z [n, H_q * r] (head h's latents at columns h r .. h r + r - 1).
    """
    X = np.asarray(X, np.float64)
    A = np.asarray(A_heads, np.float64)
    n, Hq, d = X.shape
    r = A.shape[2]
    Z = np.empty((n, Hq * r))
    for h in range(Hq):
        Z[:, h * r:(h + 1) * r] = X[:, h, :] @ A[h // group]
    return Z


def staged_decoder(A_heads, num_q_heads: int):
    """D = blockdiag_h(A_{g(h)}^T), [H_q r, H_q d]: each head decoded by its own
    up-projection B_v = A_v^T."""
    A = np.asarray(A_heads, np.float64)
    H_kv, d, r = A.shape
    group = num_q_heads // H_kv
    D = np.zeros((num_q_heads * r, num_q_heads * d))
    for h in range(num_q_heads):
        D[h * r:(h + 1) * r, h * d:(h + 1) * d] = A[h // group].T
    return D


def fit_joint_decoder(X, A_heads, group: int):
    """Decoder of the complete attention output from the latents of every
    partition: D = argmin_D |X - Z D|_F^2 (numpy least squares on the
    samples), X flattened to [n, H_q d]. Returns D [H_q r, H_q d]."""
    X = np.asarray(X, np.float64)
    n = X.shape[0]
    Z = latent_outputs(X, A_heads, group)
    D, *_ = np.linalg.lstsq(Z, X.reshape(n, -1), rcond=None)
    return D


def fit_partition_decoders(X, A_heads, group: int, partitions):
    """Each partition fitted in isolation: partition p (a list of KV heads)
    decodes its own query heads' outputs from its own latents only, by least
    squares; D is block diagonal over the partitions."""
    X = np.asarray(X, np.float64)
    n, Hq, d = X.shape
    Z = latent_outputs(X, A_heads, group)
    r = Z.shape[1] // Hq
    D = np.zeros((Hq * r, Hq * d))
    for part in partitions:
        heads = [h for g in part for h in range(g * group, (g + 1) * group)]
        zc = np.concatenate([np.arange(h * r, (h + 1) * r) for h in heads])
        xc = np.concatenate([np.arange(h * d, (h + 1) * d) for h in heads])
        Dp, *_ = np.linalg.lstsq(Z[:, zc], X.reshape(n, -1)[:, xc], rcond=None)
        D[np.ix_(zc, xc)] = Dp
    return D


def fold_decoder(W_o, D):
    """F = W_o D^T: the output projection seen from the latents of all heads,
    [hidden, H_q r] (with the staged D this is fold_output_weights)."""
    return np.asarray(W_o, np.float64) @ np.asarray(D, np.float64).T


def complete_output_error(X, A_heads, group: int, D, W_o):
    """sum_n |W_o x_n - W_o D^T z_n|^2: the loss on the complete output."""
    X = np.asarray(X, np.float64)
    n = X.shape[0]
    Z = latent_outputs(X, A_heads, group)
    R = (X.reshape(n, -1) - Z @ np.asarray(D, np.float64)) @ np.asarray(W_o, np.float64).T
    return float(np.sum(R * R))
