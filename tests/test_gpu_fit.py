"""GPU parity of the factor fit (kvlr_fit_moments, kvlr_fit_factors).

The argument has three links, each checked here or on the CPU:
  1. the GPU's float64 moments equal the exact moments of the same samples
     within the float32 summation bound (n + 2) * 2^-24 * |X|^T |Y|
     (elementwise; bf16 products are exact, f32 products round once);
  2. kvlr_fit_factors writes exactly RNE(kvlr_fit_solve(those moments)) in
     the storage type (bit-exact; the host solve is pinned to the oracle's
     fit to 1e-10 on the CPU, tests/test_fit_host.py);
  3. end to end, the factors match the oracle's float64 fit of the samples
     within bf16 rounding (2^-8 relative) plus 2e-4 absolute: the moments'
     relative error is at most about 1e-6 and the smallest relative
     eigenvalue gap of the samples about 3e-2, so eigenvectors move by about
     3e-5. W_pred = (v^T v)^-1 v^T K also amplifies the moment error by the
     condition number kappa = lam_v[0] / lam_v[-1] of v^T v (about 46 at
     r_v = 64, 2300 at r_v = 128 for these spectra), so its absolute slack
     is (2e-4 + 2e-6 kappa) times its largest entry.
"""

import numpy as np
import pytest
import torch

from decode_attention_rank_amd import _lib as K
from decode_attention_rank_amd import synth
from decode_attention_rank_amd.fit import FactorFit
from decode_attention_rank_amd.workloads import DEFAULT_FIT_WORKLOAD, FIT_WORKLOADS
from oracle import fit_factors

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def _wl(**kw):
    return FIT_WORKLOADS[DEFAULT_FIT_WORKLOAD].scaled(**kw)


CASES = [
    (dict(), 5000),                                                              # 2 runs, ragged
    (dict(head_dim=64, rank_v=16, rank_k=16, shared_rank=8, num_kv_heads=2, num_q_heads=8), 777),
    (dict(key_mode="latent", rank_k=64, shared_rank=0, num_kv_heads=3, num_q_heads=6), 4200),
    (dict(head_dim=64, rank_v=32, rank_k=16, shared_rank=16, num_kv_heads=2, num_q_heads=4,
          storage="f32"), 3001),
    (dict(key_mode="latent", rank_k=32, shared_rank=0, num_kv_heads=1, num_q_heads=4,
          storage="f32"), 2500),
    (dict(rank_v=128, rank_k=16, shared_rank=32, num_kv_heads=2, num_q_heads=8), 4100),  # r_v = d
    # one full 64-token stage (no tail); ranks well below n so the residual is defined
    (dict(num_kv_heads=1, num_q_heads=8, rank_v=16, rank_k=16, shared_rank=8), 64),
]
IDS = ["d128-bf16-exact", "d64-bf16-exact", "d128-bf16-latent", "d64-f32-exact", "d128-f32-latent",
       "rv128-bf16", "one-stage"]


def _exact_moments(k, v):
    """float64 moments and their float32 summation bounds, per head: [H, 3, d, d]."""
    n, H, d = k.shape
    M = np.empty((H, 3, d, d))
    B = np.empty((H, 3, d, d))
    for g in range(H):
        vv = v[:, g].double().cpu().numpy()
        kk = k[:, g].double().cpu().numpy()
        for m, (X, Y) in enumerate(((vv, vv), (kk, kk), (vv, kk))):
            M[g, m] = X.T @ Y
            B[g, m] = (n + 2) * U32 * (np.abs(X).T @ np.abs(Y))
    return M, B


def _storage(x, wl):
    t = torch.from_numpy(np.ascontiguousarray(x)).float()
    return t.to(torch.bfloat16) if wl.storage == "bf16" else t


def _check_moments(Mg, M, B, what):
    err = np.abs(Mg - M)
    worst = (err / (B + 1e-300)).max()
    print(f"  {what}: max |err| / bound = {worst:.3g}", flush=True)
    assert np.all(err <= B), what


def _check_end_to_end(fit, k, v, heads):
    wl = fit.wl
    rnd = 2.0 ** -8 if wl.storage == "bf16" else 2.0 ** -23
    got = {n: t.float().cpu().numpy() for n, t in fit.factors().items() if t is not None}
    for g in heads:
        ref = fit_factors(k[:, g].double().cpu().numpy(), v[:, g].double().cpu().numpy(),
                          wl.rank_v, wl.rank_k, key_mode=wl.key_mode)
        for name in ("A_v", "A_k", "W_pred"):
            if ref[name] is None:
                continue
            if name == "W_pred":
                kappa = ref["lam_v"][0] / ref["lam_v"][-1]
                scale = np.abs(ref[name]).max() * (1.0 + 1e-2 * kappa)
            else:
                scale = 1.0
            err = np.abs(got[name][g] - ref[name])
            tol = rnd * np.abs(ref[name]) + 2e-4 * scale
            print(f"  head {g} {name}: max err {err.max():.3g} (scale {scale:.3g})", flush=True)
            assert np.all(err <= tol), (g, name)
        np.testing.assert_allclose(got["B_v"][g], got["A_v"][g].T, rtol=0, atol=0)
        np.testing.assert_allclose(got["B_k"][g], got["A_k"][g].T, rtol=0, atol=0)
        np.testing.assert_allclose(fit.lam_v[g], ref["lam_v"], rtol=1e-4)
        np.testing.assert_allclose(fit.lam_k[g], ref["lam_k"], rtol=1e-4, atol=1e-5 * ref["lam_k"][0])


@pytest.mark.parametrize("kw,n", CASES, ids=IDS)
def test_fit_matches_moments_solve_and_oracle(kw, n):
    wl = _wl(**kw)
    print("case", wl.head_dim, wl.rank_v, wl.rank_k, wl.storage, wl.key_mode, wl.num_kv_heads, n,
          flush=True)
    k, v = synth.make_fit_samples(wl, n, device="cuda")
    fit = FactorFit(wl, n)
    H, d = wl.num_kv_heads, wl.head_dim
    Md = torch.empty(H, 3, d, d, dtype=torch.float64, device="cuda")
    fit.moments(k, v, n, Md, 0)
    torch.cuda.synchronize()
    Mg = Md.cpu().numpy()
    M, B = _exact_moments(k, v)
    _check_moments(Mg, M, B, "moments")
    # link 2: the factors are RNE of the host solve of these moments
    fit.fit(k, v)
    torch.cuda.synchronize()
    A_v, A_k = np.zeros((H, d, wl.rank_v)), np.zeros((H, d, wl.rank_k))
    W = np.zeros((H, wl.rank_v, d)) if wl.exact else None
    K.kvlr_fit_solve(fit.shape, np.ascontiguousarray(Mg), A_v, A_k, W)
    pairs = [(A_v, fit.A_v), (A_v.transpose(0, 2, 1), fit.B_v), (A_k, fit.A_k),
             (A_k.transpose(0, 2, 1), fit.B_k)]
    if wl.exact:
        pairs.append((W, fit.W_pred))
    for want, have in pairs:
        assert torch.equal(_storage(want, wl), have.cpu())
    # link 3: end to end against the oracle's fit
    _check_end_to_end(fit, k, v, range(H))


def test_moments_accumulate_and_empty_batches():
    wl = _wl(num_kv_heads=2, num_q_heads=8, head_dim=64, rank_v=16, rank_k=16, shared_rank=8)
    n, n1 = 6000, 2300
    k, v = synth.make_fit_samples(wl, n, device="cuda")
    fit = FactorFit(wl, n)
    Md = torch.empty(2, 3, 64, 64, dtype=torch.float64, device="cuda")
    fit.moments(k, v, n1, Md, 0)
    fit.moments(k[n1:], v[n1:], n - n1, Md, 1)
    fit.moments(k, v, 0, Md, 1)            # n = 0 adds nothing
    torch.cuda.synchronize()
    M, B = _exact_moments(k, v)
    _check_moments(Md.cpu().numpy(), M, B, "accumulated")
    fit.moments(k, v, 0, Md, 0)            # n = 0 without accumulate zeroes
    torch.cuda.synchronize()
    assert torch.count_nonzero(Md).item() == 0


def test_rank_deficient_samples_report_numerical_error():
    wl = _wl(num_kv_heads=1, num_q_heads=4, head_dim=64, rank_v=32, rank_k=16, shared_rank=8)
    k, v = synth.make_fit_samples(wl, 20, device="cuda")
    fit = FactorFit(wl, 20)
    with pytest.raises(K.KvlrError) as e:
        fit.fit(k, v)
    assert e.value.status == K.KVLR_ERR_NUMERICAL


def test_full_size_fit_workload():
    """The calibration workload at full size (one sample per cached token of
    the 8B routed cache), in the configuration the benchmark times; the
    oracle checks the first and last KV heads."""
    wl = FIT_WORKLOADS[DEFAULT_FIT_WORKLOAD]
    n = synth.fit_sample_count(wl)
    print("case", wl.name, n, flush=True)
    k, v = synth.make_fit_samples(wl, n, device="cuda")
    fit = FactorFit(wl, n)
    fit.fit(k, v)
    torch.cuda.synchronize()
    Mg = fit.workspace[: wl.num_kv_heads * 3 * wl.head_dim ** 2 * 8].view(torch.float64)
    Mg = Mg.view(wl.num_kv_heads, 3, wl.head_dim, wl.head_dim).cpu().numpy()
    heads = [0, wl.num_kv_heads - 1]
    for g in heads:
        M, B = _exact_moments(k[:, g:g + 1], v[:, g:g + 1])
        _check_moments(Mg[g:g + 1], M, B, f"head {g} moments")
    _check_end_to_end(fit, k, v, heads)
