"""Host half of the factor fit: kvlr_fit_solve (float64 eigen-solves and the
least-squares key prediction inside the library) against the oracle's fit,
given moments formed in float64 from seeded calibration samples. CPU only:
kvlr_fit_solve touches no device.

The two sides share nothing but the samples: the library reduces to
tridiagonal form and runs shifted QR steps, the oracle calls numpy's eigh and
solve on the samples themselves. The sample spectra decay geometrically
(distinct eigenvalues), so eigenvectors are unique up to sign, and both sides
fix the sign the same way (largest-magnitude entry positive).
"""

import os

import numpy as np
import pytest

from decode_attention_rank_amd import _lib as K
from decode_attention_rank_amd import synth
from decode_attention_rank_amd.fit import fit_shape
from decode_attention_rank_amd.workloads import DEFAULT_FIT_WORKLOAD, FIT_WORKLOADS
import oracle as O
from oracle import fit_factors


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(K.LIB_PATH):
        from decode_attention_rank_amd import build
        build.build(verbose=False)
    return K.lib()


def _wl(**kw):
    return FIT_WORKLOADS[DEFAULT_FIT_WORKLOAD].scaled(**kw)


def _samples(wl, n):
    Kt, Vt = synth.make_fit_samples(wl, n)
    return Kt.double().numpy(), Vt.double().numpy()


def _moments(Ks, Vs):
    n, H, d = Ks.shape
    M = np.empty((H, 3, d, d))
    for g in range(H):
        v, k = Vs[:, g], Ks[:, g]
        M[g, 0], M[g, 1], M[g, 2] = v.T @ v, k.T @ k, v.T @ k
    return M


def _host_solve(wl, M):
    H, d, rv, rk = wl.num_kv_heads, wl.head_dim, wl.rank_v, wl.rank_k
    out = dict(A_v=np.zeros((H, d, rv)), A_k=np.zeros((H, d, rk)),
               W_pred=np.zeros((H, rv, d)) if wl.exact else None,
               lam_v=np.zeros((H, rv)), lam_k=np.zeros((H, rk)))
    K.kvlr_fit_solve(fit_shape(wl), np.ascontiguousarray(M), out["A_v"], out["A_k"], out["W_pred"],
                     out["lam_v"], out["lam_k"])
    return out


CASES = [
    dict(),                                                        # d 128, r 64/32, exact
    dict(head_dim=64, rank_v=16, rank_k=16, shared_rank=8, num_kv_heads=2, num_q_heads=8),
    dict(key_mode="latent", rank_k=64, shared_rank=0, num_kv_heads=3, num_q_heads=6),
    dict(head_dim=64, rank_v=64, rank_k=32, shared_rank=16, num_kv_heads=1, num_q_heads=4,
         storage="f32"),                                           # r_v = d: v carries all of V
]


@pytest.mark.parametrize("kw", CASES, ids=["d128-exact", "d64-exact", "d128-latent", "rv-eq-d"])
def test_host_solve_matches_oracle(lib, kw):
    wl = _wl(**kw)
    Ks, Vs = _samples(wl, 3000)
    got = _host_solve(wl, _moments(Ks, Vs))
    for g in range(wl.num_kv_heads):
        ref = fit_factors(Ks[:, g], Vs[:, g], wl.rank_v, wl.rank_k, key_mode=wl.key_mode)
        np.testing.assert_allclose(got["lam_v"][g], ref["lam_v"], rtol=1e-9)
        np.testing.assert_allclose(got["lam_k"][g], ref["lam_k"], rtol=1e-8,
                                   atol=1e-9 * ref["lam_k"][0])
        # eigenvalue gaps of the samples are a few percent: vectors agree closely
        np.testing.assert_allclose(got["A_v"][g], ref["A_v"], atol=1e-10)
        np.testing.assert_allclose(got["A_k"][g], ref["A_k"], atol=1e-10)
        if wl.exact:
            W = ref["W_pred"]
            np.testing.assert_allclose(got["W_pred"][g], W, atol=1e-10 * np.abs(W).max())
        else:
            assert np.all(got["lam_k"][g][:-1] >= got["lam_k"][g][1:])


def test_host_solve_orthonormal_and_sign_convention(lib):
    wl = _wl(num_kv_heads=2, num_q_heads=8)
    Ks, Vs = _samples(wl, 2000)
    got = _host_solve(wl, _moments(Ks, Vs))
    for g in range(2):
        for A in (got["A_v"][g], got["A_k"][g]):
            np.testing.assert_allclose(A.T @ A, np.eye(A.shape[1]), atol=1e-12)
            big = np.abs(A).argmax(axis=0)
            assert np.all(A[big, np.arange(A.shape[1])] > 0)
        assert np.all(np.diff(got["lam_v"][g]) <= 0)


def test_moments_accumulate_linearly(lib):
    """Moments of two batches added equal the moments of the union: the fit of
    the union equals the fit of summed moments (what streaming calibration
    relies on)."""
    wl = _wl(num_kv_heads=1, num_q_heads=4, head_dim=64, rank_v=16, rank_k=16, shared_rank=8)
    Ks, Vs = _samples(wl, 2400)
    M = _moments(Ks[:1000], Vs[:1000]) + _moments(Ks[1000:], Vs[1000:])
    got = _host_solve(wl, M)
    ref = fit_factors(Ks[:, 0], Vs[:, 0], 16, 16, key_mode="exact")
    np.testing.assert_allclose(got["A_v"][0], ref["A_v"], atol=1e-10)
    np.testing.assert_allclose(got["W_pred"][0], ref["W_pred"], atol=1e-10 * np.abs(ref["W_pred"]).max())


def test_rank_deficient_samples_are_rejected(lib):
    wl = _wl(num_kv_heads=1, num_q_heads=4, head_dim=64, rank_v=32, rank_k=16, shared_rank=8)
    Ks, Vs = _samples(wl, 20)  # fewer samples than rank_v: v^T v is singular
    with pytest.raises(K.KvlrError) as e:
        _host_solve(wl, _moments(Ks, Vs))
    assert e.value.status == K.KVLR_ERR_NUMERICAL
    # latent keys need no least-squares solve: the same samples still fit
    _host_solve(wl.scaled(key_mode="latent", shared_rank=0), _moments(Ks, Vs))


def test_diagonal_moments_give_coordinate_axes(lib):
    """Diagonal moments with distinct entries: the eigenvectors are the
    coordinate axes in decreasing order of the entries (a closed form)."""
    wl = _wl(num_kv_heads=1, num_q_heads=1, head_dim=64, rank_v=16, rank_k=16, key_mode="latent",
             shared_rank=0)
    rng = np.random.default_rng(3)
    dv, dk = rng.permutation(64) + 1.0, rng.permutation(64) + 0.5
    M = np.zeros((1, 3, 64, 64))
    M[0, 0] = np.diag(dv)
    M[0, 1] = np.diag(dk)
    got = _host_solve(wl, M)
    for diag, A, lam in ((dv, got["A_v"][0], got["lam_v"][0]), (dk, got["A_k"][0], got["lam_k"][0])):
        order = np.argsort(-diag)[:16]
        np.testing.assert_allclose(lam, diag[order], rtol=1e-14)
        np.testing.assert_allclose(A, np.eye(64)[:, order], atol=1e-14)


def test_choose_residual_ranks_cases_and_library(lib):
    from oracle import choose_residual_ranks
    # hand-made spectra: energy within the top 64 = 100 units
    lam = np.zeros((4, 64))
    lam[0, :16] = 100 / 16                   # all of it in the first 16
    lam[1, :32] = 100 / 32                   # half in 0..15, half in 16..31
    lam[2, :] = 100 / 64                     # flat: 25 % per 16
    lam[3, :16] = 89 / 16
    lam[3, 16:] = 11 / 48                    # 89 % in the first 16
    assert choose_residual_ranks(lam, 0.9) == [16, 32, 64, 32]
    assert choose_residual_ranks(lam, 0.5) == [16, 16, 32, 16]
    # r_max 32: head 3 keeps 89 of 92.7 units in its top 16 (96 %)
    assert choose_residual_ranks(lam[:, :32], 0.9) == [16, 32, 32, 16]
    s = fit_shape(_wl(num_kv_heads=4, num_q_heads=16, rank_k=64))
    assert K.kvlr_choose_residual_ranks(s, np.ascontiguousarray(lam), 0.9) == [16, 32, 64, 32]
    rng = np.random.default_rng(9)
    for frac in (0.5, 0.8, 0.95, 1.0):
        lam = -np.sort(-rng.exponential(size=(4, 64)) * rng.uniform(0.05, 1, (4, 1)) ** 8, axis=1)
        assert K.kvlr_choose_residual_ranks(s, np.ascontiguousarray(lam), frac) == \
            choose_residual_ranks(lam, frac)


# ----------------------------------------------------------------------------
# Joint decoder fit: the library's host solve against the oracle's
# least-squares fit on the samples (CPU only)
# ----------------------------------------------------------------------------

def _joint_case(seed, Hq, H_kv, d, r, n):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((n, 8))
    X = np.empty((n, Hq, d))
    for h in range(Hq):
        M = rng.standard_normal((8, d)) / np.sqrt(8)
        X[:, h] = (s + 0.5 * rng.standard_normal((n, 8))) @ M
    X += 0.05 * rng.standard_normal(X.shape)
    A = np.stack([np.linalg.qr(rng.standard_normal((d, d)))[0][:, :r] for _ in range(H_kv)])
    return X, A


@pytest.mark.parametrize("Hq,H_kv,d,r,n", [(4, 2, 64, 16, 300), (8, 1, 128, 32, 700), (8, 8, 64, 16, 500)])
def test_joint_solve_matches_the_oracle_least_squares(Hq, H_kv, d, r, n):
    X, A = _joint_case(41, Hq, H_kv, d, r, n)
    Z = O.latent_outputs(X, A, Hq // H_kv)
    zz = Z.T @ Z
    zx = Z.T @ X.reshape(n, -1)
    shape = K.make_shape(num_q_heads=Hq, num_kv_heads=H_kv, head_dim=d, page_size=64, rank_v=r,
                         rank_k=16, dtype=K.KVLR_DTYPE_BF16, key_mode=K.KVLR_KEYS_EXACT,
                         num_phys_pages=1)
    D = K.kvlr_fit_joint_solve(shape, zz, zx)
    ref = O.fit_joint_decoder(X, A, Hq // H_kv)
    cond = np.linalg.cond(zz)
    assert np.abs(D - ref).max() <= 1e-13 * cond * np.abs(ref).max() + 1e-12


def test_joint_solve_rejects_undetermined_latents():
    X, A = _joint_case(42, 4, 2, 64, 16, 40)   # 40 samples, 64 latents
    Z = O.latent_outputs(X, A, 2)
    shape = K.make_shape(num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=64, rank_v=16,
                         rank_k=16, dtype=K.KVLR_DTYPE_BF16, key_mode=K.KVLR_KEYS_EXACT,
                         num_phys_pages=1)
    with pytest.raises(K.KvlrError) as e:
        K.kvlr_fit_joint_solve(shape, Z.T @ Z, Z.T @ X.reshape(40, -1))
    assert e.value.status == K.KVLR_ERR_NUMERICAL
