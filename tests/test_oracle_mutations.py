"""Each test plants one plausible mistake in the oracle (on the CPU, by
monkeypatching) and checks that at least one pin catches it."""

import numpy as np
import pytest

import oracle
import oracle.kvlr_oracle as K
import tests.test_oracle_pins as pins


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(K, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _fails(test_fn, *args):
    with pytest.raises(AssertionError):
        test_fn(*args)


def test_residual_sign_flip_is_caught(monkeypatch):
    def wrong(v, c, W_pred, B_k):
        return np.asarray(v, float) @ np.asarray(W_pred, float) - np.asarray(c, float) @ np.asarray(B_k, float)
    _patch(monkeypatch, "key_approximation", wrong)
    _fails(pins.test_page_scores_match_explicit_loops)


def test_transposed_query_projection_is_caught(monkeypatch):
    def wrong(q_group, W_pred, B_k):
        q = np.asarray(q_group, float)
        return q @ np.asarray(W_pred, float).T, q @ np.asarray(B_k, float).T[::-1]
    _patch(monkeypatch, "project_queries", wrong)
    _fails(pins.test_latent_space_scores_equal_decompressed_scores)


def test_truncating_bf16_is_caught(monkeypatch):
    def wrong(x):
        x = np.asarray(x, np.float32)
        b = x.view(np.uint32) & np.uint32(0xFFFF0000)
        return b.view(np.float32).astype(np.float64)
    _patch(monkeypatch, "round_bf16", wrong)
    _fails(pins.test_round_bf16_matches_torch_rne)


def test_ties_to_higher_index_is_caught(monkeypatch):
    def wrong(S, k):
        order = sorted(range(len(S)), key=lambda j: (-float(S[j]), -j))
        return sorted(order[:k])
    _patch(monkeypatch, "select_top_pages", wrong)
    _fails(pins.test_topk_matches_subset_enumeration, 0)


def test_residual_against_unrounded_latent_is_caught(monkeypatch):
    real = K.encode_tokens

    def wrong(Kn, Vn, A_v, A_k, W_pred=None, *, key_mode, storage):
        out = real(Kn, Vn, A_v, A_k, W_pred, key_mode=key_mode, storage=storage)
        if key_mode == "exact":
            v_raw = np.asarray(Vn, float) @ np.asarray(A_v, float)
            out["k_lat"] = K.round_to_storage((np.asarray(Kn, float) - v_raw @ np.asarray(W_pred, float))
                                              @ np.asarray(A_k, float), storage)
        return out
    _patch(monkeypatch, "encode_tokens", wrong)
    _fails(pins.test_residual_uses_stored_value_latent)


def test_missing_max_subtraction_scale_is_caught(monkeypatch):
    real = K.attend

    def wrong(q_group, keys, v_rows, B_v, scale):
        return real(q_group, keys, v_rows, B_v, 1.0)   # drops the softmax scale
    _patch(monkeypatch, "attend", wrong)
    _fails(pins.test_full_rank_dense_equals_sdpa, "f64", 1e-12)


def test_page_score_mean_instead_of_max_is_caught(monkeypatch):
    def wrong(q_group, v, c, W_pred, B_k, L, P):
        N = -(-L // P)
        Kt = K.key_approximation(np.asarray(v)[:L], np.asarray(c)[:L], W_pred, B_k)
        s = np.asarray(q_group, float) @ Kt.T
        return np.array([s[:, j * P:min((j + 1) * P, L)].mean() for j in range(N)])
    _patch(monkeypatch, "page_scores", wrong)
    _fails(pins.test_page_scores_full_rank_residual_are_exact_key_scores)


def test_off_by_one_length_is_caught(monkeypatch):
    def wrong(pages, L, P):
        out = []
        for j in pages:
            out.extend(range(j * P, min((j + 1) * P, L + 1)))
        return np.asarray(out, dtype=np.int64)
    _patch(monkeypatch, "tokens_of_pages", wrong)
    _fails(pins.test_tokens_past_length_are_ignored)


def test_wrong_k_rounding_is_caught(monkeypatch):
    def wrong(N, num, den):
        return 0 if N <= 0 else min(N, max(1, (N * num) // den))
    _patch(monkeypatch, "pages_to_keep", wrong)
    _fails(pins.test_pages_to_keep, 9, 1, 8, 2)


def test_untransposed_fold_is_caught(monkeypatch):
    # folding with B_v instead of its transpose (it runs when r_v = d)
    def bad(B_v_heads, W_o):
        B = np.asarray(B_v_heads, np.float64)
        W = np.asarray(W_o, np.float64)
        n, _, d = B.shape
        return np.concatenate([W[:, h * d:(h + 1) * d] @ B[h] for h in range(n)], axis=1)
    _patch(monkeypatch, "fold_output_weights", bad)
    _fails(pins.test_fold_equals_library_linear_of_upprojected_outputs, 16)


def test_fit_residual_taken_from_the_keys_is_caught(monkeypatch):
    # principal directions of K instead of the prediction's residual
    good = K.fit_factors

    def bad(Kx, Vx, r_v, r_k, *, key_mode):
        out = good(Kx, Vx, r_v, r_k, key_mode=key_mode)
        lam, A = K._top_eigvecs(np.asarray(Kx, np.float64).T @ np.asarray(Kx, np.float64), r_k)
        out.update(A_k=A, B_k=A.T.copy(), lam_k=lam)
        return out
    _patch(monkeypatch, "fit_factors", bad)
    _fails(pins.test_fit_residual_basis_is_the_residual_principal_subspace)


def test_fit_smallest_directions_is_caught(monkeypatch):
    def bad_top(C, r):
        w, U = np.linalg.eigh(np.asarray(C, np.float64))
        return w[:r], U[:, :r]
    monkeypatch.setattr(K, "_top_eigvecs", bad_top)
    _fails(pins.test_fit_value_basis_is_the_top_right_singular_subspace)


def test_latents_from_the_wrong_kv_head_are_caught(monkeypatch):
    def wrong(X, A_heads, group):
        X = np.asarray(X, float)
        A = np.asarray(A_heads, float)
        n, Hq, d = X.shape
        r = A.shape[2]
        return np.concatenate([X[:, h] @ A[h % A.shape[0]] for h in range(Hq)], axis=1)
    _patch(monkeypatch, "latent_outputs", wrong)
    _fails(pins.test_latent_outputs_use_each_heads_kv_encoder)


def test_joint_fit_done_head_by_head_is_caught(monkeypatch):
    # a "joint" fit that ignores the other heads' latents (per-head decoders)
    def wrong(X, A_heads, group):
        X = np.asarray(X, float)
        n, Hq, d = X.shape
        return K.fit_partition_decoders(X, A_heads, group,
                                        [[g] for g in range(np.asarray(A_heads).shape[0])])
    _patch(monkeypatch, "fit_joint_decoder", wrong)
    _fails(pins.test_joint_fit_never_loses_to_isolated_or_staged_decoders, 35)


def test_decoder_fitted_against_the_latents_transposed_is_caught(monkeypatch):
    def wrong(X, A_heads, group):
        X = np.asarray(X, float)
        n = X.shape[0]
        Z = K.latent_outputs(X, A_heads, group)
        # the encoder-side map (x -> z) instead of the decoder (z -> x)
        E, *_ = np.linalg.lstsq(X.reshape(n, -1), Z, rcond=None)
        return E.T
    _patch(monkeypatch, "fit_joint_decoder", wrong)
    _fails(pins.test_joint_decoder_satisfies_the_normal_equations)
