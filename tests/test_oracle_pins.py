"""Pins of the CPU oracle against facts fixed outside the oracle itself:
library routines (torch's bfloat16 conversion, torch's scaled-dot-product
attention), closed forms, brute force on tiny inputs, and a hand-derived
worked example. Runs on the CPU only.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _orth(rng, d):
    q, r = np.linalg.qr(rng.standard_normal((d, d)))
    return q * np.sign(np.diag(r))


# ----------------------------------------------------------------------------
# Storage rounding
# ----------------------------------------------------------------------------

def test_round_bf16_known_values():
    # bfloat16 spacing on [1, 2) is 2**-7.
    assert O.round_bf16(1.0) == 1.0
    assert O.round_bf16(1 + 2 ** -8) == 1.0                 # tie -> even (1.0)
    assert O.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6     # tie -> even (k = 2)
    assert O.round_bf16(1 + 2 ** -8 + 2 ** -20) == 1 + 2 ** -7
    assert O.round_bf16(-(1 + 3 * 2 ** -8)) == -(1 + 2 ** -6)
    assert O.round_bf16(2.0 ** -133) == 2.0 ** -133         # smallest subnormal
    assert O.round_bf16(3.5e38) == np.inf                   # beyond max finite
    assert np.isnan(O.round_bf16(np.nan))


def test_round_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
    ])
    # exact ties: bfloat16 values plus half a spacing
    base = torch.from_numpy(rng.standard_normal(4000).astype(np.float32)).to(torch.bfloat16)
    bits = base.view(torch.int16).to(torch.int32) & 0xFFFF
    tie = ((bits << 16) | 0x8000).to(torch.int32).view(torch.float32).numpy()
    x = np.concatenate([x, tie])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_round_fp8_e4m3_known_values():
    # OCP 8-bit floating point, E4M3: largest normal S.1111.110 = 448, smallest
    # normal S.0001.000 = 2**-6, largest subnormal S.0000.111 = 0.875 * 2**-6,
    # smallest subnormal S.0000.001 = 2**-9; spacing on [1, 2) is 2**-3.
    R = O.round_fp8_e4m3
    assert R(448.0) == 448.0
    assert R(2.0 ** -6) == 2.0 ** -6
    assert R(0.875 * 2.0 ** -6) == 0.875 * 2.0 ** -6
    assert R(2.0 ** -9) == 2.0 ** -9
    assert R(1 + 2 ** -4) == 1.0                  # tie -> even (1.0)
    assert R(1 + 3 * 2 ** -4) == 1.25             # tie -> even (k = 2)
    assert R(1 + 2 ** -4 + 2 ** -10) == 1.125
    assert R(-(1 + 3 * 2 ** -4)) == -1.25
    assert R(2.0 ** -10) == 0.0                   # half the smallest subnormal -> 0
    assert R(3 * 2.0 ** -10) == 2.0 ** -8         # tie between 1 and 2 subnormal units -> 2
    assert R(464.0) == 448.0                      # tie with 480 (not a finite value) -> 448
    assert R(465.0) == 448.0 and R(1e6) == 448.0 and R(-1e6) == -448.0   # saturation
    assert R(np.inf) == 448.0 and R(-np.inf) == -448.0
    assert np.isnan(R(np.nan))


def test_round_fp8_e4m3_matches_torch_inside_the_range():
    """torch's float32 -> float8_e4m3fn conversion rounds to nearest even and
    maps magnitudes from 464 up to NaN; inside (-464, 464) the two agree."""
    rng = np.random.default_rng(5)
    parts = [rng.standard_normal(20000) * sc for sc in (1e-3, 0.1, 1.0, 30.0)]
    parts.append(rng.uniform(-463.0, 463.0, 5000))
    x = np.concatenate(parts).astype(np.float32)
    vals = torch.arange(127, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    vals = vals.to(torch.float64).numpy()       # codes 0..126: every finite value >= 0
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact ties
    x = np.concatenate([x, mids, -mids])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.round_fp8_e4m3(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_round_fp8_e4m3_fixes_every_code():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    codes = codes.to(torch.float64).numpy()
    assert np.isnan(codes).sum() == 2          # S.1111.111 only
    fin = codes[~np.isnan(codes)]
    np.testing.assert_array_equal(O.round_fp8_e4m3(fin), fin)
    assert fin.max() == 448.0 and np.abs(fin[fin != 0]).min() == 2.0 ** -9


def test_round_to_storage_f32_is_ieee_single():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(1000)
    np.testing.assert_array_equal(O.round_to_storage(x, "f32"), x.astype(np.float32).astype(np.float64))
    np.testing.assert_array_equal(O.round_to_storage(x, "f64"), x)


# ----------------------------------------------------------------------------
# Check (1): rank r = head_dim with orthonormal factors is textbook attention
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("storage,tol", [("f64", 1e-12), ("f32", 2e-6)])
def test_full_rank_dense_equals_sdpa(storage, tol):
    rng = np.random.default_rng(2)
    d, L, P, G = 16, 37, 8, 3
    Qv, Qk = _orth(rng, d), _orth(rng, d)
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    q = rng.standard_normal((G, d))
    st = O.empty_state(L, d, d, d, "latent")
    st = O.append_tokens(st, 0, K, V, Qv, Qk, key_mode="latent", storage=storage)
    f = {"B_v": Qv.T, "B_k": Qk.T}
    res = O.decode_pair(q, st, f, L, P, key_mode="latent")
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :],
        torch.from_numpy(K)[None, None].expand(1, G, L, d),
        torch.from_numpy(V)[None, None].expand(1, G, L, d))[0, :, 0, :].numpy()
    np.testing.assert_allclose(res["o"], ref, atol=tol, rtol=0)
    # the up-projection of z is the same output
    np.testing.assert_allclose(O.upproject(res["z"], Qv.T), ref, atol=tol, rtol=0)
    assert res["sel"] == list(range(-(-L // P)))


def test_full_rank_encode_roundtrip():
    rng = np.random.default_rng(3)
    d = 32
    A = _orth(rng, d)
    V = rng.standard_normal((50, d))
    enc = O.encode_tokens(V, V, A, A, key_mode="latent", storage="f64")
    np.testing.assert_allclose(enc["v"] @ A.T, V, atol=1e-12)
    np.testing.assert_allclose(enc["k_lat"] @ A.T, V, atol=1e-12)


def test_inputs_in_factor_span_roundtrip_at_low_rank():
    rng = np.random.default_rng(4)
    d, r = 64, 16
    A = _orth(rng, d)[:, :r]
    V = rng.standard_normal((20, r)) @ A.T          # inside span(A)
    enc = O.encode_tokens(V, V, A, A, key_mode="latent", storage="f64")
    np.testing.assert_allclose(enc["v"] @ A.T, V, atol=1e-12)


# ----------------------------------------------------------------------------
# Check (2): routing that keeps every page equals dense exact-key attention
# ----------------------------------------------------------------------------

def _routed_case(rng, d=16, r_v=8, r_k=6, L=45, G=2, storage="bf16"):
    A_v = _orth(rng, d)[:, :r_v]
    W = rng.standard_normal((r_v, d)) * 0.3
    A_k = _orth(rng, d)[:, :r_k]
    K = O.round_bf16(rng.standard_normal((L, d)))
    V = O.round_bf16(rng.standard_normal((L, d)))
    q = rng.standard_normal((G, d)) / math.sqrt(d)
    st = O.empty_state(L, d, r_v, r_k, "exact")
    st = O.append_tokens(st, 0, K, V, A_v, A_k, W, key_mode="exact", storage=storage)
    f = {"B_v": A_v.T, "B_k": A_k.T, "W_pred": W}
    return q, st, f, K, V


def test_route_all_pages_equals_dense_exact_attention():
    rng = np.random.default_rng(5)
    q, st, f, K, V = _routed_case(rng)
    L, P = 45, 8
    res = O.decode_pair(q, st, f, L, P, key_mode="exact", topk=(1, 1))
    assert res["sel"] == list(range(6))
    # independent textbook computation with torch in float64
    s = torch.from_numpy(q) @ torch.from_numpy(K).T / math.sqrt(q.shape[1])
    w = torch.softmax(s, dim=-1)
    z = (w @ torch.from_numpy(st["v"][:L])).numpy()
    o = (w @ (torch.from_numpy(st["v"][:L]) @ torch.from_numpy(f["B_v"]))).numpy()
    np.testing.assert_allclose(res["z"], z, atol=1e-12)
    np.testing.assert_allclose(res["o"], o, atol=1e-12)
    np.testing.assert_allclose(res["lse"], torch.logsumexp(s, -1).numpy(), atol=1e-12)


def test_route_k1_attends_one_page_only():
    rng = np.random.default_rng(6)
    q, st, f, K, V = _routed_case(rng)
    L, P = 45, 8
    res = O.decode_pair(q, st, f, L, P, key_mode="exact", topk=(1, 6))
    assert len(res["sel"]) == 1
    j = res["sel"][0]
    assert j == int(np.argmax(res["scores"]))
    t = np.arange(j * P, min((j + 1) * P, L))
    s = q @ K[t].T / math.sqrt(q.shape[1])
    w = np.exp(s - s.max(1, keepdims=True))
    w /= w.sum(1, keepdims=True)
    np.testing.assert_allclose(res["z"], w @ st["v"][t], atol=1e-12)


# ----------------------------------------------------------------------------
# Check (3): brute force over page scores and over k-subsets
# ----------------------------------------------------------------------------

def _brute_force_topk(S, k):
    """The unique k-subset with no outside page that beats an inside page
    under (higher score, then lower index)."""
    N = len(S)
    winners = []
    for sub in itertools.combinations(range(N), k):
        inside = set(sub)
        ok = True
        for a in inside:
            for b in range(N):
                if b in inside:
                    continue
                if S[b] > S[a] or (S[b] == S[a] and b < a):
                    ok = False
        if ok:
            winners.append(list(sub))
    assert len(winners) == 1
    return winners[0]


@pytest.mark.parametrize("seed", range(12))
def test_topk_matches_subset_enumeration(seed):
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(1, 10))
    S = rng.integers(-3, 4, size=N).astype(np.float64)  # many exact ties
    for k in range(0, N + 1):
        assert O.select_top_pages(S, k) == _brute_force_topk(S, k)


def test_page_scores_match_explicit_loops():
    rng = np.random.default_rng(7)
    d, r_v, r_k, L, P, G = 5, 3, 2, 11, 4, 2
    v = rng.standard_normal((L + 3, r_v))
    c = rng.standard_normal((L + 3, r_k))
    W = rng.standard_normal((r_v, d))
    B = rng.standard_normal((r_k, d))
    q = rng.standard_normal((G, d))
    S = O.page_scores(q, v, c, W, B, L, P)
    N = -(-L // P)
    assert S.shape == (N,)
    for j in range(N):
        best = -math.inf
        for t in range(j * P, min(j * P + P, L)):
            for h in range(G):
                acc = 0.0
                for i in range(d):
                    kt = sum(v[t, a] * W[a, i] for a in range(r_v)) + sum(c[t, b] * B[b, i] for b in range(r_k))
                    acc += q[h, i] * kt
                best = max(best, acc)
        assert abs(S[j] - best) < 1e-12


def test_page_scores_full_rank_residual_are_exact_key_scores():
    rng = np.random.default_rng(8)
    d, r_v, L, P, G = 12, 4, 30, 7, 3
    A_v = _orth(rng, d)[:, :r_v]
    W = rng.standard_normal((r_v, d))
    A_k = _orth(rng, d)                    # r_k = d, orthonormal
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    q = rng.standard_normal((G, d))
    st = O.append_tokens(O.empty_state(L, d, r_v, d, "exact"), 0, K, V, A_v, A_k, W,
                         key_mode="exact", storage="f64")
    S = O.page_scores(q, st["v"], st["k_lat"], W, A_k.T, L, P)
    raw = q @ K.T
    want = [raw[:, j * P:min(j * P + P, L)].max() for j in range(-(-L // P))]
    np.testing.assert_allclose(S, want, atol=1e-11)


def test_latent_space_scores_equal_decompressed_scores():
    rng = np.random.default_rng(9)
    d, r_v, r_k, L, G = 16, 6, 5, 20, 4
    v = rng.standard_normal((L, r_v))
    c = rng.standard_normal((L, r_k))
    W = rng.standard_normal((r_v, d))
    B = rng.standard_normal((r_k, d))
    q = rng.standard_normal((G, d))
    qh, qt = O.project_queries(q, W, B)
    latent = qh @ v.T + qt @ c.T
    decompressed = q @ O.key_approximation(v, c, W, B).T
    np.testing.assert_allclose(latent, decompressed, atol=1e-11)


# ----------------------------------------------------------------------------
# Closed forms and special cases
# ----------------------------------------------------------------------------

def test_zero_query_gives_mean_latent():
    rng = np.random.default_rng(10)
    q, st, f, K, V = _routed_case(rng)
    q = np.zeros_like(q)
    L, P = 45, 8
    res = O.decode_pair(q, st, f, L, P, key_mode="exact", topk=(1, 2))
    t = O.tokens_of_pages(res["sel"], L, P)
    np.testing.assert_allclose(res["z"], np.broadcast_to(st["v"][t].mean(0), res["z"].shape), atol=1e-12)
    np.testing.assert_allclose(res["lse"], math.log(len(t)), atol=1e-12)


def test_single_token_output_is_decompressed_value():
    rng = np.random.default_rng(11)
    d, r = 8, 4
    A = _orth(rng, d)[:, :r]
    K = rng.standard_normal((1, d))
    V = rng.standard_normal((1, d))
    st = O.append_tokens(O.empty_state(1, d, r, r, "latent"), 0, K, V, A, A,
                         key_mode="latent", storage="f64")
    res = O.decode_pair(rng.standard_normal((2, d)), st, {"B_v": A.T, "B_k": A.T}, 1, 16, key_mode="latent")
    np.testing.assert_allclose(res["o"], np.broadcast_to(st["v"][0] @ A.T, (2, d)), atol=1e-12)
    np.testing.assert_allclose(res["z"], np.broadcast_to(st["v"][0], (2, r)), atol=1e-12)


def test_empty_context():
    st = O.empty_state(0, 8, 4, 4, "exact")
    f = {"B_v": np.eye(4, 8), "B_k": np.eye(4, 8), "W_pred": np.zeros((4, 8))}
    res = O.decode_pair(np.ones((2, 8)), st, f, 0, 16, key_mode="exact", topk=(1, 8))
    assert res["sel"] == []
    assert np.all(res["z"] == 0) and np.all(res["o"] == 0)
    assert np.all(np.isneginf(res["lse"]))


def test_upproject_orthonormal_rows_preserve_norm():
    rng = np.random.default_rng(12)
    B = _orth(rng, 32)[:, :8].T      # 8 orthonormal rows
    z = rng.standard_normal((5, 8))
    o = O.upproject(z, B)
    np.testing.assert_allclose(np.linalg.norm(o, axis=1), np.linalg.norm(z, axis=1), rtol=1e-12)


def test_tokens_past_length_are_ignored():
    rng = np.random.default_rng(13)
    q, st, f, K, V = _routed_case(rng, L=45)
    L, P = 41, 8                      # last page holds one valid token
    res = O.decode_pair(q, st, f, L, P, key_mode="exact", topk=(1, 2))
    st2 = {k: a.copy() for k, a in st.items()}
    for k in st2:
        st2[k][L:] = 1e6              # garbage beyond the length
    res2 = O.decode_pair(q, st2, f, L, P, key_mode="exact", topk=(1, 2))
    assert res["sel"] == res2["sel"]
    np.testing.assert_array_equal(res["z"], res2["z"])
    # last page's score is the score of its single valid token
    Kt = O.key_approximation(st["v"][40:41], st["k_lat"][40:41], f["W_pred"], f["B_k"])
    assert abs(res["scores"][5] - (q @ Kt.T).max()) < 1e-12
    # every page kept: the garbage rows must not enter the softmax
    res3 = O.decode_pair(q, st2, f, L, P, key_mode="exact", topk=(1, 1))
    s = q @ K[:L].T / np.sqrt(q.shape[1])
    w = np.exp(s - s.max(1, keepdims=True))
    w /= w.sum(1, keepdims=True)
    np.testing.assert_allclose(res3["z"], w @ st["v"][:L], atol=1e-12)


def test_residual_uses_stored_value_latent():
    # identity factors: v = round(V), c = round(K - round(V)).
    x = 1 + 2 ** -9                    # not a bfloat16 value; rounds to 1.0
    K = np.array([[x, 0.0]])
    V = np.array([[x, 0.0]])
    eye = np.eye(2)
    enc = O.encode_tokens(K, V, eye, eye, eye, key_mode="exact", storage="bf16")
    assert enc["v"][0, 0] == 1.0
    assert enc["k_lat"][0, 0] == 2 ** -9
    np.testing.assert_array_equal(enc["k_exact"], K)


def test_perfect_prediction_gives_zero_residual():
    rng = np.random.default_rng(14)
    d, r_v, r_k = 16, 8, 4
    A_v = _orth(rng, d)[:, :r_v]
    W = rng.standard_normal((r_v, d))
    A_k = _orth(rng, d)[:, :r_k]
    V = rng.standard_normal((10, d))
    K = (V @ A_v) @ W
    enc = O.encode_tokens(K, V, A_v, A_k, W, key_mode="exact", storage="f64")
    np.testing.assert_allclose(enc["k_lat"], 0.0, atol=1e-12)


@pytest.mark.parametrize("N,num,den,k", [
    (0, 1, 8, 0), (1, 1, 8, 1), (7, 1, 8, 1), (8, 1, 8, 1), (9, 1, 8, 2),
    (512, 1, 8, 64), (2048, 1, 16, 128), (513, 1, 8, 65), (5, 1, 1, 5), (5, 3, 2, 5)])
def test_pages_to_keep(N, num, den, k):
    assert O.pages_to_keep(N, num, den) == k


def test_chunked_append_equals_one_shot():
    rng = np.random.default_rng(15)
    d, r_v, r_k, n = 16, 8, 4, 23
    A_v = _orth(rng, d)[:, :r_v]
    W = rng.standard_normal((r_v, d))
    A_k = _orth(rng, d)[:, :r_k]
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    one = O.append_tokens(O.empty_state(0, d, r_v, r_k, "exact"), 0, K, V, A_v, A_k, W,
                          key_mode="exact", storage="bf16")
    st = O.empty_state(0, d, r_v, r_k, "exact")
    for a, b in [(0, 5), (5, 6), (6, 17), (17, 23)]:
        st = O.append_tokens(st, a, K[a:b], V[a:b], A_v, A_k, W, key_mode="exact", storage="bf16")
    for name in one:
        np.testing.assert_array_equal(one[name], st[name])


# ----------------------------------------------------------------------------
# Hand-derived worked example (tests/golden/worked_example.json)
# ----------------------------------------------------------------------------

def test_golden_worked_example():
    with open(os.path.join(HERE, "golden", "worked_example.json")) as fh:
        g = json.load(fh)
    inp, exp = g["inputs"], g["expected"]
    q = np.array(inp["q"])
    K = np.array([[math.log(a), 0.0] for a in inp["keys_ln_arg"]])
    v = np.array(inp["v"])
    L, P, scale = 3, inp["page_size"], inp["scale"]
    eye = np.eye(2)
    lat = {"v": v, "k_lat": K}
    res = O.decode_pair(q, lat, {"B_v": eye, "B_k": eye}, L, P, key_mode="latent", scale=scale)
    np.testing.assert_allclose(res["z"], exp["latent"]["z"], atol=1e-12)
    np.testing.assert_allclose(res["o"], exp["latent"]["o"], atol=1e-12)
    np.testing.assert_allclose(np.exp(res["lse"]), exp["latent"]["lse_exp"], rtol=1e-12)
    routed = {"v": v, "k_lat": K, "k_exact": K}
    f = {"B_v": eye, "B_k": eye, "W_pred": np.zeros((2, 2))}
    for key, kk in (("routed_k1", (1, 3)), ("routed_k2", (2, 3))):
        res = O.decode_pair(q, routed, f, L, P, key_mode="exact", scale=scale, topk=kk)
        assert res["sel"] == exp[key]["sel"]
        np.testing.assert_allclose(res["z"], exp[key]["z"], atol=1e-12)
        np.testing.assert_allclose(np.exp(res["lse"]), exp[key]["lse_exp"], rtol=1e-12)
    res = O.decode_pair(q, routed, f, L, P, key_mode="exact", scale=scale, topk=(1, 3))
    np.testing.assert_allclose(np.exp(res["scores"]), exp["routed_k1"]["scores_exp"], rtol=1e-12)


# ----------------------------------------------------------------------------
# Output projection and its fold onto the value latents
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("r_v", [8, 16])
def test_fold_equals_library_linear_of_upprojected_outputs(r_v):
    rng = np.random.default_rng(21)
    n_heads, d, hidden = 6, 16, 40
    B_v = rng.standard_normal((n_heads, r_v, d))
    W_o = rng.standard_normal((hidden, n_heads * d))
    z = rng.standard_normal((n_heads, r_v))
    # library path: o_h = z_h B_v[h] by torch matmul, then nn.functional.linear
    zt = torch.from_numpy(z).unsqueeze(1)                       # [H, 1, r_v]
    o = torch.bmm(zt, torch.from_numpy(B_v).contiguous()).reshape(1, -1)
    ref = torch.nn.functional.linear(o, torch.from_numpy(W_o)).reshape(-1).numpy()
    F = O.fold_output_weights(B_v, W_o)
    assert F.shape == (hidden, n_heads * r_v)
    np.testing.assert_allclose(O.latent_output_projection(z, F), ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.output_projection(o.numpy().reshape(n_heads, d), W_o), ref,
                               rtol=1e-12, atol=1e-12)


def test_fold_with_identity_upprojection_is_the_output_weight():
    rng = np.random.default_rng(22)
    n_heads, d, hidden = 3, 8, 12
    B_v = np.stack([np.eye(d)] * n_heads)
    W_o = rng.standard_normal((hidden, n_heads * d))
    np.testing.assert_array_equal(O.fold_output_weights(B_v, W_o), W_o)


def test_fold_column_is_one_latent_direction():
    # a unit latent e_(h, e) is carried by column h*r_v + e of F, which is the
    # output weight applied to row e of that head's up-projection
    rng = np.random.default_rng(23)
    n_heads, d, r_v, hidden = 4, 8, 4, 10
    B_v = rng.standard_normal((n_heads, r_v, d))
    W_o = rng.standard_normal((hidden, n_heads * d))
    F = O.fold_output_weights(B_v, W_o)
    for h in range(n_heads):
        for e in range(r_v):
            col = np.zeros(hidden)
            for n in range(hidden):
                col[n] = sum(W_o[n, h * d + j] * B_v[h, e, j] for j in range(d))
            np.testing.assert_allclose(F[:, h * r_v + e], col, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# Factor fitting
# ----------------------------------------------------------------------------

def _fit_data(rng, n=600, d=16, rs=6, ns=3, noise=0.01):
    """Values of rank rs (distinct scales) plus noise; keys share ns of the
    value coefficients and carry rs - ns of their own."""
    Qv, Qk = _orth(rng, d), _orth(rng, d)
    scale = 1.0 + 0.7 * np.arange(rs)[::-1]
    C = rng.standard_normal((n, rs)) * scale
    E = rng.standard_normal((n, rs - ns)) * (1.0 + 0.5 * np.arange(rs - ns)[::-1])
    V = C @ Qv[:, :rs].T + noise * rng.standard_normal((n, d))
    K = np.concatenate([C[:, :ns], E], axis=1) @ Qk[:, :rs].T + noise * rng.standard_normal((n, d))
    return K, V


def test_fit_value_basis_is_the_top_right_singular_subspace():
    rng = np.random.default_rng(31)
    K, V = _fit_data(rng)
    f = O.fit_factors(K, V, 6, 4, key_mode="exact")
    _, _, Vt = np.linalg.svd(V, full_matrices=False)   # library routine
    P_ref = Vt[:6].T @ Vt[:6]
    np.testing.assert_allclose(f["A_v"] @ f["A_v"].T, P_ref, atol=1e-9)
    np.testing.assert_allclose(f["A_v"].T @ f["A_v"], np.eye(6), atol=1e-12)
    np.testing.assert_allclose(f["B_v"], f["A_v"].T)


def test_fit_prediction_is_least_squares():
    rng = np.random.default_rng(32)
    K, V = _fit_data(rng)
    f = O.fit_factors(K, V, 6, 4, key_mode="exact")
    v = V @ f["A_v"]
    W_ls, *_ = np.linalg.lstsq(v, K, rcond=None)         # library routine
    np.testing.assert_allclose(f["W_pred"], W_ls, atol=1e-9)


def test_fit_residual_basis_is_the_residual_principal_subspace():
    rng = np.random.default_rng(33)
    K, V = _fit_data(rng)
    f = O.fit_factors(K, V, 6, 3, key_mode="exact")
    R = K - (V @ f["A_v"]) @ f["W_pred"]
    _, _, Vt = np.linalg.svd(R, full_matrices=False)
    np.testing.assert_allclose(f["A_k"] @ f["A_k"].T, Vt[:3].T @ Vt[:3], atol=1e-9)
    # the residual of the prediction is orthogonal to the value latents
    np.testing.assert_allclose((V @ f["A_v"]).T @ R, 0, atol=1e-8)


def test_fit_recovers_an_exact_structure():
    # noise-free: values of rank r_v; keys = shared part through a known map plus
    # a part of rank r_k orthogonal to it -> prediction and residual are exact
    rng = np.random.default_rng(34)
    n, d, rv, rk = 400, 12, 4, 3
    Q = _orth(rng, d)
    C = rng.standard_normal((n, rv)) * np.array([4.0, 3.0, 2.0, 1.0])
    V = C @ Q[:, :rv].T
    M = rng.standard_normal((rv, d))
    E = rng.standard_normal((n, rk)) * np.array([3.0, 2.0, 1.0])
    K = C @ M + E @ Q[:, rv:rv + rk].T
    f = O.fit_factors(K, V, rv, rk, key_mode="exact")
    v = V @ f["A_v"]
    R = K - v @ f["W_pred"]
    # what the latents predict plus the rank-r_k residual reconstruct K exactly
    np.testing.assert_allclose(v @ f["W_pred"] + (R @ f["A_k"]) @ f["B_k"], K, atol=1e-9)
    np.testing.assert_allclose(f["A_v"] @ f["A_v"].T @ V.T, V.T, atol=1e-9)


def test_fit_latent_mode_uses_key_principal_directions():
    rng = np.random.default_rng(35)
    K, V = _fit_data(rng)
    f = O.fit_factors(K, V, 6, 5, key_mode="latent")
    assert f["W_pred"] is None
    _, _, Vt = np.linalg.svd(K, full_matrices=False)
    np.testing.assert_allclose(f["A_k"] @ f["A_k"].T, Vt[:5].T @ Vt[:5], atol=1e-9)


# ----------------------------------------------------------------------------
# Joint fit of the decoders across partitions (BasisKV English abstract:
# factors optimised jointly across per-GPU partitions against the complete
# attention output)
# ----------------------------------------------------------------------------

def _correlated_outputs(rng, n, Hq, d, m=8, shared=1.0, own=0.5, noise=0.05):
    """Attention-output-like samples whose heads share a hidden component:
    x_h = (shared s_n + own u_{n,h}) M_h + noise."""
    s = rng.standard_normal((n, m))
    X = np.empty((n, Hq, d))
    for h in range(Hq):
        M = rng.standard_normal((m, d)) / math.sqrt(m)
        X[:, h] = (shared * s + own * rng.standard_normal((n, m))) @ M
    return X + noise * rng.standard_normal(X.shape)


def _encoders(rng, H_kv, d, r):
    return np.stack([_orth(rng, d)[:, :r] for _ in range(H_kv)])


def test_joint_decoder_at_full_rank_is_the_staged_decoder():
    # r = d with orthonormal encoders: z A^T = x exactly, so the unique least-
    # squares decoder is blockdiag(A^T) and the complete output is exact
    rng = np.random.default_rng(31)
    Hq, H_kv, d = 4, 2, 8
    X = _correlated_outputs(rng, 200, Hq, d)
    A = _encoders(rng, H_kv, d, d)
    D = O.fit_joint_decoder(X, A, Hq // H_kv)
    assert np.allclose(D, O.staged_decoder(A, Hq), atol=1e-10)
    W = rng.standard_normal((12, Hq * d))
    assert O.complete_output_error(X, A, Hq // H_kv, D, W) < 1e-18 * np.sum(X * X)


def test_joint_decoder_of_outputs_in_the_latent_span_is_the_staged_decoder():
    # x_h = c_h A_g^T (outputs inside each head's encoder span): Z = C and
    # X = Z blockdiag(A^T) exactly, a unique fit when Z has full column rank
    rng = np.random.default_rng(32)
    Hq, H_kv, d, r, n = 6, 3, 16, 4, 100
    A = _encoders(rng, H_kv, d, r)
    C = rng.standard_normal((n, Hq, r))
    X = np.stack([C[:, h] @ A[h // 2].T for h in range(Hq)], axis=1)
    D = O.fit_joint_decoder(X, A, Hq // H_kv)
    assert np.allclose(D, O.staged_decoder(A, Hq), atol=1e-10)


def test_joint_decoder_satisfies_the_normal_equations():
    # the residual of a least-squares fit is orthogonal to every regressor
    rng = np.random.default_rng(33)
    Hq, H_kv, d, r = 8, 2, 16, 4
    X = _correlated_outputs(rng, 300, Hq, d)
    A = _encoders(rng, H_kv, d, r)
    Z = O.latent_outputs(X, A, Hq // H_kv)
    R = X.reshape(300, -1) - Z @ O.fit_joint_decoder(X, A, Hq // H_kv)
    assert np.abs(Z.T @ R).max() < 1e-9 * np.abs(Z).max() * np.abs(X).max() * 300


def test_latent_outputs_use_each_heads_kv_encoder():
    rng = np.random.default_rng(34)
    Hq, H_kv, d, r = 4, 2, 8, 3
    X = rng.standard_normal((5, Hq, d))
    A = _encoders(rng, H_kv, d, r)
    Z = O.latent_outputs(X, A, 2)
    for n in range(5):
        for h in range(Hq):
            for j in range(r):
                assert abs(Z[n, h * r + j] - sum(X[n, h, i] * A[h // 2, i, j] for i in range(d))) < 1e-12


@pytest.mark.parametrize("seed", [35, 36])
def test_joint_fit_never_loses_to_isolated_or_staged_decoders(seed):
    # joint, isolated and staged decoders are all feasible for the joint
    # problem; isolated decoders contain the staged ones. On heads sharing a
    # hidden component the joint one is strictly better, for any W_o.
    rng = np.random.default_rng(seed)
    Hq, H_kv, d, r = 8, 4, 16, 4
    X = _correlated_outputs(rng, 400, Hq, d)
    A = _encoders(rng, H_kv, d, r)
    parts = [[0, 1], [2, 3]]
    W = rng.standard_normal((24, Hq * d))
    e_joint = O.complete_output_error(X, A, 2, O.fit_joint_decoder(X, A, 2), W)
    e_iso = O.complete_output_error(X, A, 2, O.fit_partition_decoders(X, A, 2, parts), W)
    e_staged = O.complete_output_error(X, A, 2, O.staged_decoder(A, Hq), W)
    assert e_joint < 0.95 * e_iso
    assert e_iso <= e_staged * (1 + 1e-12)


def test_joint_fit_equals_isolated_fits_when_partitions_never_co_occur():
    # each sample has output in one partition only: the cross-partition
    # moments vanish and the joint problem splits into the isolated ones
    rng = np.random.default_rng(37)
    Hq, H_kv, d, r, n = 4, 2, 12, 3, 240
    X = _correlated_outputs(rng, n, Hq, d)
    X[: n // 2, 2:] = 0.0   # partition 1 (KV head 1: heads 2, 3) silent
    X[n // 2:, :2] = 0.0    # partition 0 silent
    A = _encoders(rng, H_kv, d, r)
    Dj = O.fit_joint_decoder(X, A, 2)
    Di = O.fit_partition_decoders(X, A, 2, [[0], [1]])
    assert np.allclose(Dj, Di, atol=1e-9)


def test_folded_staged_decoder_is_the_output_projection_fold():
    rng = np.random.default_rng(38)
    Hq, H_kv, d, r = 4, 2, 8, 4
    A = _encoders(rng, H_kv, d, r)
    W = rng.standard_normal((16, Hq * d))
    B_v_heads = np.stack([A[h // 2].T for h in range(Hq)])
    assert np.allclose(O.fold_decoder(W, O.staged_decoder(A, Hq)),
                       O.fold_output_weights(B_v_heads, W), atol=1e-12)
