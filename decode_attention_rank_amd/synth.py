"""Seeded synthetic inputs for the decode workloads.

This module only draws random numbers and arranges them; it holds none of
the method's arithmetic (no encode, no routing, no attention). Both the HIP
path and the CPU oracle consume what it produces.

Recipe (per KV head g; all draws seeded by (workload seed, role, sequence)):
  * Two orthonormal bases Q_v[g], Q_k[g] of R^d (QR of a seeded Gaussian,
    float64 on the host, signs fixed so the R diagonal is positive). With
    value_basis "identity" Q_v is the identity, so full-rank value factors
    store the values themselves (the uncompressed reference).
  * Signal coefficients per token: C ~ N(0,1) of width signal_rank for V;
    key coefficients kc = [C[:, :shared_rank], E] with E ~ N(0,1), so the
    first shared_rank key coordinates are carried by the value (the part a
    V-latent key prediction can recover). Dense workloads use shared_rank 0
    (independent keys).
  * Raw tokens (appended on the step): V = C Q_v[:, :rs]^T + s*N,
    K = kc Q_k[:, :rs]^T + s*N, rounded to the storage type.
  * Pre-existing cache tokens are drawn directly in latent coordinates, the
    coordinates a rank-r projection onto the same bases would give: V latent
    v = [C, 0] + s*N (width rank_v); routed key residual c = [E, 0] + s*N
    (width rank_k); dense key latent k = [kc, 0] + s*N; original key
    K = kc Q_k[:, :rs]^T + s*N. All rounded to the storage type.
  * Latents are stored in the workload's latent type (bf16, f32, or FP8
    E4M3 with bf16 keys and factors).
  * Factors: A_v = Q_v[:, :rank_v], B_v = A_v^T. Routed: W_pred rows
    i < shared_rank are Q_k[:, i]^T (zero below), A_k =
    Q_k[:, shared_rank:shared_rank + rank_k], B_k = A_k^T. Dense:
    A_k = Q_k[:, :rank_k], B_k = A_k^T. Rounded to the storage type.
  * Queries q ~ N(0, 1/d) per coordinate, float32.
  * Output projection W_o [hidden][H_q d] ~ N(0, 1/(H_q d)), in the storage
    type (hidden = H_q d unless the workload names its share's width).
  * Planted pages (routing signal): a seeded fraction of each sequence's
    pages get their key coefficients (and the shared value coefficients)
    shifted by boost * u, u the unit vector of Q_k[:, :rs]^T q_bar, q_bar the
    mean query of the KV group.
  * Calibration samples for the factor fit (make_fit_samples): per KV head,
    coefficients C ~ N(0,1) of full width d scaled by FIT_DECAY^i, so the
    sample spectra have distinct, geometrically spaced eigenvalues;
    V = (C * scale) Q_v^T; K = [C[:, :ns] * scale[:ns], E * FIT_KEY_SCALE *
    scale[ns:]] Q_k^T with E ~ N(0,1) (ns = shared_rank: the key part the
    value carries). No further noise. Rounded to the storage type.
  * Attention-output samples for the joint decoder fit (make_output_samples):
    per sample n a hidden vector s_n ~ N(0, diag(OUT_DECAY^i)) of width
    OUT_HIDDEN shared by every query head, and per head
    x_h = (s_n + OUT_OWN u_{n,h}) M_h + OUT_NOISE e, with u, e ~ N(0, I) and
    M_h ~ N(0, 1/OUT_HIDDEN) [OUT_HIDDEN, d] seeded per head: heads of
    different KV heads (different GPUs' partitions) are correlated through
    s_n, as outputs of heads reading one residual stream are. float32.
  * Ragged contexts: L ~ round(lognormal(mu, sigma)) clipped to
    [ctx_min, ctx_max], mu = mean of the log bounds, sigma = quarter of the
    log range.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from .workloads import Workload

_ROLE = {"bases": 1, "q": 2, "coef": 3, "noise": 4, "lens": 5, "planted": 6,
         "pages": 7, "raw": 8, "oproj": 9, "fit": 10, "outputs": 11}

FIT_DECAY = 0.97      # per-coordinate scale ratio of the calibration samples
OUT_HIDDEN = 64       # width of the hidden part the attention-output samples share
OUT_DECAY = 0.97      # its per-coordinate scale ratio
OUT_OWN = 0.5         # head-specific part, relative
OUT_NOISE = 0.05      # isotropic noise
FIT_KEY_SCALE = 0.8   # key-only coordinates relative to the shared ones

TORCH_STORAGE = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.float8_e4m3fn}


def _seed(wl_seed: int, role: str, *idx: int) -> int:
    s = np.random.SeedSequence([wl_seed, _ROLE[role], *idx])
    return int(s.generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)


def _gen(device, wl_seed: int, role: str, *idx: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(wl_seed, role, *idx))
    return g


def storage_dtype(wl: Workload) -> torch.dtype:
    return TORCH_STORAGE[wl.storage]


def latent_dtype(wl: Workload) -> torch.dtype:
    """Type of the stored latents (torch's float32 -> float8 conversion rounds
    to nearest even; synthetic latents stay far inside the E4M3 range)."""
    return TORCH_STORAGE[wl.lat_storage]


def bases(wl: Workload):
    """Orthonormal (Q_v, Q_k) per KV head, float64 on the host: [H_kv, d, d] each."""
    g = _gen("cpu", wl.seed, "bases")
    d = wl.head_dim
    out = []
    for _ in range(2):
        m = torch.randn(wl.num_kv_heads, d, d, generator=g, dtype=torch.float64)
        q, r = torch.linalg.qr(m)
        sign = torch.sign(torch.diagonal(r, dim1=-2, dim2=-1))
        sign[sign == 0] = 1.0
        out.append(q * sign.unsqueeze(-2))
    if wl.value_basis == "identity":
        out[0] = torch.eye(d, dtype=torch.float64).expand(wl.num_kv_heads, d, d).clone()
    return out[0], out[1]


def make_factors(wl: Workload, device="cpu"):
    """Factor tensors in the storage type: A_v [H,d,r_v], B_v [H,r_v,d],
    A_k [H,d,r_k], B_k [H,r_k,d], W_pred [H,r_v,d] (routed only, else None)."""
    Qv, Qk = bases(wl)
    H, d, rv, rk, ns = wl.num_kv_heads, wl.head_dim, wl.rank_v, wl.rank_k, wl.shared_rank
    A_v = Qv[:, :, :rv]
    if wl.exact:
        if ns > rv or ns + rk > d:
            raise ValueError("shared_rank must fit in rank_v and shared_rank + rank_k in head_dim")
        W = torch.zeros(H, rv, d, dtype=torch.float64)
        W[:, :ns, :] = Qk[:, :, :ns].transpose(1, 2)
        A_k = Qk[:, :, ns:ns + rk]
    else:
        W = None
        A_k = Qk[:, :, :rk]
    dt = storage_dtype(wl)

    def st(x):
        return None if x is None else x.contiguous().to(dt).to(device)

    return {
        "A_v": st(A_v), "B_v": st(A_v.transpose(1, 2)),
        "A_k": st(A_k), "B_k": st(A_k.transpose(1, 2)), "W_pred": st(W),
    }


def make_queries(wl: Workload, device="cpu") -> torch.Tensor:
    g = _gen("cpu", wl.seed, "q")
    q = torch.randn(wl.batch, wl.num_q_heads, wl.head_dim, generator=g, dtype=torch.float64)
    return (q / math.sqrt(wl.head_dim)).to(torch.float32).to(device)


def output_width(wl: Workload) -> int:
    """Output features of the attention layer (the head share's row count of W_o)."""
    return wl.hidden if wl.hidden else wl.num_q_heads * wl.head_dim


def make_output_weight(wl: Workload, device="cpu") -> torch.Tensor:
    """Output projection W_o [hidden][H_q * d] in the storage type, entries
    N(0, 1 / (H_q d)) (seeded)."""
    g = _gen("cpu", wl.seed, "oproj")
    n_in = wl.num_q_heads * wl.head_dim
    W = torch.randn(output_width(wl), n_in, generator=g, dtype=torch.float64) / math.sqrt(n_in)
    return W.to(storage_dtype(wl)).to(device)


def make_seq_lens(wl: Workload) -> list[int]:
    """Context length of each sequence after the step's append."""
    if not wl.ragged:
        return [wl.context] * wl.batch
    rng = np.random.default_rng(_seed(wl.seed, "lens"))
    lo, hi = math.log(wl.ctx_min), math.log(wl.ctx_max)
    mu, sigma = 0.5 * (lo + hi), 0.25 * (hi - lo)
    L = np.rint(rng.lognormal(mu, sigma, wl.batch)).astype(np.int64)
    return [int(x) for x in np.clip(L, wl.ctx_min, wl.ctx_max)]


def make_page_table(wl: Workload, seq_lens, spare_pages: int = 0):
    """Seeded scattered page allocation.

    Returns (page_table int32 [B, max_pages] with -1 beyond each sequence's
    pages, num_phys_pages). Physical page ids are a random permutation.
    """
    P = wl.page_size
    n_pages = [-(-L // P) for L in seq_lens]
    max_pages = max(1, max(n_pages))
    total = sum(n_pages) + spare_pages
    g = _gen("cpu", wl.seed, "pages")
    perm = torch.randperm(max(total, 1), generator=g).to(torch.int32)
    pt = torch.full((wl.batch, max_pages), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(n_pages):
        pt[b, :n] = perm[off:off + n]
        off += n
    return pt, max(total, 1)


def planted_pages(wl: Workload, b: int, n_pages: int) -> torch.Tensor:
    """Seeded set of planted logical pages of sequence b (may be empty)."""
    if wl.planted_frac <= 0 or n_pages == 0:
        return torch.zeros(0, dtype=torch.int64)
    m = math.ceil(wl.planted_frac * n_pages)
    g = _gen("cpu", wl.seed, "planted", b)
    return torch.sort(torch.randperm(n_pages, generator=g)[:m]).values


def _planted_direction(wl: Workload, Qk_g: torch.Tensor, q_group: torch.Tensor) -> torch.Tensor:
    qbar = q_group.to(torch.float64).mean(dim=0).cpu()
    w = Qk_g[:, :wl.signal_rank].T @ qbar
    return (w / w.norm()).to(torch.float32)


def _coefficients(wl: Workload, b: int, g: int, pos0: int, n: int, device, Qk, q):
    """Signal coefficients of tokens pos0 .. pos0+n-1 of sequence b, head g."""
    rs, ns = wl.signal_rank, wl.shared_rank
    gen = _gen(device, wl.seed, "coef", b, g, pos0)
    C = torch.randn(n, rs, generator=gen, device=device)
    E = torch.randn(n, rs - ns, generator=gen, device=device)
    kc = torch.cat([C[:, :ns], E], dim=1)
    if wl.planted_frac > 0 and n > 0:
        pages = planted_pages(wl, b, -(-make_seq_lens(wl)[b] // wl.page_size))
        if pages.numel():
            pos = torch.arange(pos0, pos0 + n)
            mask = torch.isin(pos // wl.page_size, pages).to(device)
            G = wl.group
            u = _planted_direction(wl, Qk[g], q[b, g * G:(g + 1) * G]).to(device)
            shift = wl.planted_boost * u * mask[:, None].to(torch.float32)
            kc = kc + shift
            C = C.clone()
            C[:, :ns] += shift[:, :ns]
    return C, kc


def synth_latent_cache(wl: Workload, b: int, n: int, device="cpu", *, q=None, Qk=None):
    """Pre-existing cache of sequence b, tokens 0 .. n-1, in latent coordinates.

    Returns dict of storage-type tensors: "v" [H, n, r_v], "k_lat" [H, n, r_k]
    and, routed, "k_exact" [H, n, d]. Positions are logical token indices.
    """
    if Qk is None:
        _, Qk = bases(wl)
    if q is None:
        q = make_queries(wl)
    H, d, rv, rk, rs, ns, s = (wl.num_kv_heads, wl.head_dim, wl.rank_v, wl.rank_k,
                               wl.signal_rank, wl.shared_rank, wl.noise_std)
    dt = storage_dtype(wl)
    lt = latent_dtype(wl)
    v = torch.empty(H, n, rv, dtype=lt, device=device)
    kl = torch.empty(H, n, rk, dtype=lt, device=device)
    ke = torch.empty(H, n, d, dtype=dt, device=device) if wl.exact else None
    for g in range(H):
        C, kc = _coefficients(wl, b, g, 0, n, device, Qk, q)
        gen = _gen(device, wl.seed, "noise", b, g)
        vv = s * torch.randn(n, rv, generator=gen, device=device)
        m = min(rs, rv)
        vv[:, :m] += C[:, :m]
        v[g] = vv.to(lt)
        kk = s * torch.randn(n, rk, generator=gen, device=device)
        src = kc[:, ns:] if wl.exact else kc
        m = min(src.shape[1], rk)
        kk[:, :m] += src[:, :m]
        kl[g] = kk.to(lt)
        if wl.exact:
            basis = Qk[g, :, :rs].to(torch.float32).to(device)
            K = kc @ basis.T.contiguous() + s * torch.randn(n, d, generator=gen, device=device)
            ke[g] = K.to(dt)
    out = {"v": v, "k_lat": kl}
    if wl.exact:
        out["k_exact"] = ke
    return out


def synth_raw_tokens(wl: Workload, b: int, pos0: int, n: int, device="cpu", *, q=None,
                     Qv=None, Qk=None):
    """Raw new keys and values of sequence b at positions pos0 .. pos0+n-1.

    Returns (K, V), each [n, H_kv, d] in the storage type (token-major, the
    layout a fused QKV projection writes).
    """
    if Qv is None or Qk is None:
        Qv, Qk = bases(wl)
    if q is None:
        q = make_queries(wl)
    H, d, rs, s = wl.num_kv_heads, wl.head_dim, wl.signal_rank, wl.noise_std
    dt = storage_dtype(wl)
    K = torch.empty(n, H, d, dtype=dt, device=device)
    V = torch.empty(n, H, d, dtype=dt, device=device)
    for g in range(H):
        C, kc = _coefficients(wl, b, g, pos0, n, device, Qk, q)
        gen = _gen(device, wl.seed, "raw", b, g, pos0)
        bv = Qv[g, :, :rs].to(torch.float32).to(device)
        bk = Qk[g, :, :rs].to(torch.float32).to(device)
        V[:, g] = (C @ bv.T.contiguous() + s * torch.randn(n, d, generator=gen, device=device)).to(dt)
        K[:, g] = (kc @ bk.T.contiguous() + s * torch.randn(n, d, generator=gen, device=device)).to(dt)
    return K, V


def fit_sample_count(wl: Workload) -> int:
    """Calibration samples per KV head: every token of the workload's cache."""
    return wl.batch * wl.context


def make_fit_samples(wl: Workload, n: int, device="cpu"):
    """Calibration keys and values (K, V), each [n, H_kv, d] in the storage type."""
    Qv, Qk = bases(wl)
    H, d, ns = wl.num_kv_heads, wl.head_dim, wl.shared_rank
    dt = storage_dtype(wl)
    scale = FIT_DECAY ** torch.arange(d, dtype=torch.float64)
    kscale = scale.clone()
    kscale[ns:] *= FIT_KEY_SCALE
    scale = scale.to(torch.float32).to(device)
    kscale = kscale.to(torch.float32).to(device)
    K = torch.empty(n, H, d, dtype=dt, device=device)
    V = torch.empty(n, H, d, dtype=dt, device=device)
    for g in range(H):
        gen = _gen(device, wl.seed, "fit", g)
        C = torch.randn(n, d, generator=gen, device=device)
        E = torch.randn(n, d - ns, generator=gen, device=device)
        kc = torch.cat([C[:, :ns], E], dim=1) * kscale
        bv = Qv[g].to(torch.float32).to(device)
        bk = Qk[g].to(torch.float32).to(device)
        V[:, g] = ((C * scale) @ bv.T.contiguous()).to(dt)
        K[:, g] = (kc @ bk.T.contiguous()).to(dt)
        del C, E, kc
    return K, V


def make_output_samples(wl: Workload, n: int, device="cpu", chunk: int = 4096) -> torch.Tensor:
    """Attention-output samples X [n, H_q, d] float32 for the joint decoder fit."""
    Hq, d, m = wl.num_q_heads, wl.head_dim, OUT_HIDDEN
    gm = _gen("cpu", wl.seed, "outputs", 0)
    M = (torch.randn(Hq, m, d, generator=gm, dtype=torch.float64) / math.sqrt(m)).to(torch.float32)
    M = M.to(device)
    scale = (OUT_DECAY ** torch.arange(m, dtype=torch.float64)).to(torch.float32).to(device)
    X = torch.empty(n, Hq, d, dtype=torch.float32, device=device)
    for c0 in range(0, n, chunk):
        c = min(chunk, n - c0)
        gen = _gen(device, wl.seed, "outputs", 1, c0)
        s = torch.randn(c, m, generator=gen, device=device) * scale
        for h in range(Hq):
            u = torch.randn(c, m, generator=gen, device=device)
            e = torch.randn(c, d, generator=gen, device=device)
            X[c0:c0 + c, h] = (s + OUT_OWN * u) @ M[h] + OUT_NOISE * e
    return X
