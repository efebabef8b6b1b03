"""GPU parity of the joint decoder fit (kvlr_fit_joint_moments,
kvlr_fold_joint_decoder, kvlr_fit_joint).

Three links, each against quantities computed in float64 on the host from
the same samples and factors (never from what the GPU wrote):
  1. moments: z = x A is formed in float32 (a d-term float32 dot product,
     then the stored float32 value), so |dZ| <= (d + 2) u Zb with
     Zb = |X| |A| and u = 2^-24; the moments take float32 sums over runs of
     256 samples (257 u of sum |z_i z_j|) and float64 sums of the runs:
       |zz - Z^T Z| <= (2 (d + 2) + 258) u Zb^T Zb
       |zx - Z^T X| <= ((d + 2) + 258) u Zb^T |X|           (elementwise)
  2. solve: D = zz^-1 zx moves by at most |zz^-1|_2 (|dzx|_F + |dzz|_F |D|_F)
     for moment errors dzz, dzx within the bounds of link 1, so the GPU's D
     is compared with the oracle's least-squares D within that bound (the
     host solve alone is pinned to the oracle on the CPU,
     tests/test_fit_host.py);
  3. fold: F = W_o D^T with D in float32, float32 products summed in float32
     over runs of 256 and in float64 across runs, then rounded to bf16:
     |F - W_o D^T| <= 2^-8 |F| + 258 u |W_o| |D|^T.
End to end, the GPU's decoder lowers the complete-output loss below the
staged decoder's, as the oracle's does.
"""

import numpy as np
import pytest
import torch

import oracle as O
from decode_attention_rank_amd import _lib as K
from decode_attention_rank_amd import synth
from decode_attention_rank_amd.workloads import DEFAULT_FIT_WORKLOAD, FIT_WORKLOADS

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def _wl(Hq, Hkv, d, r, storage="bf16"):
    return FIT_WORKLOADS[DEFAULT_FIT_WORKLOAD].scaled(num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                                                       rank_v=r, rank_k=min(32, d // 2),
                                                       shared_rank=min(r, d // 4), storage=storage)


def _shape(wl):
    return K.make_shape(num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                        head_dim=wl.head_dim, page_size=64, rank_v=wl.rank_v, rank_k=wl.rank_k,
                        dtype=K.KVLR_DTYPE_BF16 if wl.storage == "bf16" else K.KVLR_DTYPE_F32,
                        key_mode=K.KVLR_KEYS_EXACT, num_phys_pages=1)


def _inputs(wl, n):
    X = synth.make_output_samples(wl, n, device="cuda")
    f = synth.make_factors(wl, "cuda")
    A = f["A_v"]
    return X, A, f


def _bounds(Xh, Ah, G):
    n, Hq, d = Xh.shape
    Zb = O.latent_outputs(np.abs(Xh), np.abs(Ah), G)
    Xa = np.abs(Xh).reshape(n, -1)
    tol_zz = (2 * (d + 2) + 258) * U32 * (Zb.T @ Zb) * 1.01
    tol_zx = ((d + 2) + 258) * U32 * (Zb.T @ Xa) * 1.01
    return tol_zz, tol_zx


CASES = [(8, 2, 64, 16, 700), (16, 4, 128, 32, 2500), (8, 8, 128, 16, 400)]


@pytest.mark.parametrize("Hq,Hkv,d,r,n", CASES)
@pytest.mark.parametrize("storage", ["bf16", "f32"])
def test_joint_moments_within_float32_bound(Hq, Hkv, d, r, n, storage):
    wl = _wl(Hq, Hkv, d, r, storage)
    print("case joint moments", Hq, Hkv, d, r, n, storage, flush=True)
    shape = _shape(wl)
    X, A, f = _inputs(wl, n)
    nl, nx = Hq * r, Hq * d
    zz = torch.empty(nl, nl, dtype=torch.float64, device="cuda")
    zx = torch.empty(nl, nx, dtype=torch.float64, device="cuda")
    ws_bytes = K.kvlr_fit_joint_workspace_bytes(shape, n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    fac = K.make_factors(**f)
    K.kvlr_fit_joint_moments(shape, fac, X, n, zz, zx, 0, ws, ws_bytes)
    torch.cuda.synchronize()
    Xh = X.double().cpu().numpy()
    Ah = A.double().cpu().numpy()
    Z = O.latent_outputs(Xh, Ah, Hq // Hkv)
    tol_zz, tol_zx = _bounds(Xh, Ah, Hq // Hkv)
    assert np.all(np.abs(zz.cpu().numpy() - Z.T @ Z) <= tol_zz)
    assert np.all(np.abs(zx.cpu().numpy() - Z.T @ Xh.reshape(n, -1)) <= tol_zx)
    # accumulate: a second call adds the same moments again
    K.kvlr_fit_joint_moments(shape, fac, X, n, zz, zx, 1, ws, ws_bytes)
    torch.cuda.synchronize()
    assert np.all(np.abs(zz.cpu().numpy() - 2 * (Z.T @ Z)) <= 2 * tol_zz)


@pytest.mark.parametrize("Hq,Hkv,d,r,n", CASES + [(32, 8, 128, 64, 8192)],
                         ids=["small", "medium", "mha", "llama3-8b-full"])
def test_joint_fit_matches_the_oracle(Hq, Hkv, d, r, n):
    wl = _wl(Hq, Hkv, d, r)
    print("case joint fit", Hq, Hkv, d, r, n, flush=True)
    shape = _shape(wl)
    X, A, f = _inputs(wl, n)
    hidden = 256
    W_o = (torch.randn(hidden, Hq * d, generator=torch.Generator().manual_seed(7)) /
           np.sqrt(Hq * d)).to(torch.bfloat16).cuda()
    nl, nx = Hq * r, Hq * d
    F = torch.empty(hidden, nl, dtype=torch.bfloat16, device="cuda")
    ws_bytes = K.kvlr_fit_joint_workspace_bytes(shape, n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    D = K.kvlr_fit_joint(shape, K.make_factors(**f), X, n, W_o, hidden, F, ws, ws_bytes, want_D=True)
    Xh = X.double().cpu().numpy()
    Ah = A.double().cpu().numpy()
    G = Hq // Hkv
    ref = O.fit_joint_decoder(Xh, Ah, G)
    # link 2: the solve's sensitivity to the moment bounds
    Z = O.latent_outputs(Xh, Ah, G)
    zz = Z.T @ Z
    tol_zz, tol_zx = _bounds(Xh, Ah, G)
    lam_min = np.linalg.eigvalsh(zz)[0]
    bound = (np.linalg.norm(tol_zx) + np.linalg.norm(tol_zz) * np.linalg.norm(ref)) / lam_min
    err = np.abs(D - ref).max()
    print(f"  D max err {err:.3e} (bound {bound:.3e}, |D| {np.abs(ref).max():.3e})", flush=True)
    assert err <= bound
    # link 3: the fold of the GPU's decoder (rounded to float32 as uploaded)
    Df = D.astype(np.float32).astype(np.float64)
    Wh = W_o.double().cpu().numpy()
    Fr = O.fold_decoder(Wh, Df)
    Fg = F.double().cpu().numpy()
    tolF = 2.0 ** -8 * np.abs(Fr) + 258 * U32 * (np.abs(Wh) @ np.abs(Df).T) + 1e-30
    assert np.all(np.abs(Fg - Fr) <= tolF * 1.01)
    # the fitted decoder beats the staged one on the complete output, as the oracle's does
    if n <= 2500:
        e_gpu = O.complete_output_error(Xh, Ah, G, D, Wh)
        e_ref = O.complete_output_error(Xh, Ah, G, ref, Wh)
        e_staged = O.complete_output_error(Xh, Ah, G, O.staged_decoder(Ah, Hq), Wh)
        assert e_gpu <= e_ref * (1 + 1e-6) and e_gpu < e_staged
