"""The seeded input generator: determinism, shapes, and that the synthetic
caches carry the structure the routing relies on (checked with the oracle)."""

import math

import numpy as np
import torch

import oracle as O
from decode_attention_rank_amd import synth
from decode_attention_rank_amd.workloads import WORKLOADS


def _small(name, **kw):
    return WORKLOADS[name].scaled(**kw)


def test_generator_is_deterministic():
    wl = _small("llama3-8b-routed-32k", batch=2, context=256)
    a = synth.synth_latent_cache(wl, 1, 200)
    b = synth.synth_latent_cache(wl, 1, 200)
    for k in a:
        assert torch.equal(a[k], b[k])
    Ka, Va = synth.synth_raw_tokens(wl, 0, 100, 7)
    Kb, Vb = synth.synth_raw_tokens(wl, 0, 100, 7)
    assert torch.equal(Ka, Kb) and torch.equal(Va, Vb)


def test_factor_shapes_and_orthonormality():
    wl = WORKLOADS["llama3-8b-routed-32k"]
    f = synth.make_factors(wl)
    H, d, rv, rk = 8, 128, 64, 32
    assert f["A_v"].shape == (H, d, rv) and f["B_v"].shape == (H, rv, d)
    assert f["A_k"].shape == (H, d, rk) and f["B_k"].shape == (H, rk, d)
    assert f["W_pred"].shape == (H, rv, d)
    A = f["A_v"][0].double()
    assert torch.allclose(A.T @ A, torch.eye(rv, dtype=torch.float64), atol=2e-2)
    assert f["A_v"].dtype == torch.bfloat16


def test_ragged_lengths_in_range():
    wl = WORKLOADS["mixed-append-routed-ragged"]
    L = synth.make_seq_lens(wl)
    assert len(L) == 32 and min(L) >= 4096 and max(L) <= 131072
    assert L == synth.make_seq_lens(wl)
    assert len(set(L)) > 10


def test_page_table_is_a_permutation():
    wl = _small("mixed-append-routed-ragged", batch=5)
    L = [1, 64, 65, 700, 4096]
    pt, n = synth.make_page_table(wl, L)
    used = pt[pt >= 0]
    assert used.numel() == sum(-(-x // 64) for x in L) == n
    assert torch.equal(torch.sort(used).values, torch.arange(n, dtype=torch.int32))


def _state(cache, g):
    return {k: cache[k][g].double().numpy() for k in cache}


def _factors_np(f, g):
    return {k: (None if f[k] is None else f[k][g].double().numpy()) for k in f}


def test_latent_cache_key_approximation_tracks_original_keys():
    wl = _small("llama3-8b-routed-32k", batch=1, context=512)
    f = synth.make_factors(wl)
    cache = synth.synth_latent_cache(wl, 0, 512)
    st, fn = _state(cache, 0), _factors_np(f, 0)
    Kt = O.key_approximation(st["v"], st["k_lat"], fn["W_pred"], fn["B_k"])
    err = np.linalg.norm(Kt - st["k_exact"]) / np.linalg.norm(st["k_exact"])
    assert err < 0.1


def test_raw_tokens_encode_to_the_latent_recipe():
    # encoding raw tokens with the oracle lands near the directly drawn latents'
    # statistics: the V latent keeps the signal, the residual the key-only part.
    wl = _small("llama3-8b-routed-32k", batch=1, context=512)
    f = synth.make_factors(wl)
    K, V = synth.synth_raw_tokens(wl, 0, 0, 256)
    fn = _factors_np(f, 0)
    enc = O.encode_tokens(K[:, 0].double().numpy(), V[:, 0].double().numpy(), fn["A_v"], fn["A_k"],
                          fn["W_pred"], key_mode="exact", storage="bf16")
    Kt = O.key_approximation(enc["v"], enc["k_lat"], fn["W_pred"], fn["B_k"])
    Kx = K[:, 0].double().numpy()
    assert np.linalg.norm(Kt - Kx) / np.linalg.norm(Kx) < 0.1
    assert abs(enc["v"][:, :48].std() - 1.0) < 0.1


def test_planted_pages_are_recalled_by_routing():
    wl = _small("llama3-70b-share-routed-128k", batch=2, context=8192)
    q = synth.make_queries(wl)
    f = synth.make_factors(wl)
    fn = _factors_np(f, 0)
    N = 8192 // 64
    recalls = []
    for b in range(2):
        cache = synth.synth_latent_cache(wl, b, 8192, q=q)
        st = _state(cache, 0)
        res = O.decode_pair(q[b, :8].double().numpy(), st, fn, 8192, 64, key_mode="exact", topk=(1, 16))
        planted = set(synth.planted_pages(wl, b, N).tolist())
        assert len(res["sel"]) == math.ceil(N / 16)
        recalls.append(len(planted & set(res["sel"])) / len(planted))
    assert min(recalls) >= 0.8


def test_output_samples_are_seeded_and_share_a_hidden_part():
    from decode_attention_rank_amd.workloads import FIT_WORKLOADS
    wl = FIT_WORKLOADS["llama3-8b-fit-512k"].scaled(num_q_heads=8, num_kv_heads=2)
    X = synth.make_output_samples(wl, 3000)
    assert X.shape == (3000, 8, wl.head_dim) and X.dtype == torch.float32
    assert torch.equal(X, synth.make_output_samples(wl, 3000))
    # heads of different KV heads are correlated through the shared hidden part:
    # the leading canonical correlation between two heads is far from zero
    a = X[:, 0].double()
    b = X[:, 7].double()
    a = a - a.mean(0)
    b = b - b.mean(0)
    qa, _ = torch.linalg.qr(a)
    qb, _ = torch.linalg.qr(b)
    assert torch.linalg.svdvals(qa.T @ qb)[0] > 0.5
