"""The C-ABI library loads, exports every function the header declares, and
rejects bad arguments on the host before touching the GPU. CPU only: no call
here reaches a kernel launch."""

import ctypes
import os
import re

import numpy as np
import pytest

from decode_attention_rank_amd import _lib as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvlr.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(K.LIB_PATH):
        from decode_attention_rank_amd import build
        build.build(verbose=False)
    return K.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(kvlr_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for fn in ("kvlr_append_encode", "kvlr_route_pages", "kvlr_decode_attn", "kvlr_upproject",
               "kvlr_project_queries"):
        assert fn in names
    assert set(names) == set(K.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert K.kvlr_version() >= 100
    assert K.kvlr_status_string(0) == "ok"
    assert "invalid" in K.kvlr_status_string(1)
    assert "unsupported" in K.kvlr_status_string(2)
    assert "workspace" in K.kvlr_status_string(3)


def _shape(**kw):
    base = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64, rank_v=64, rank_k=32,
                dtype=K.KVLR_DTYPE_BF16, key_mode=K.KVLR_KEYS_EXACT, num_phys_pages=8192)
    base.update(kw)
    return K.make_shape(**base)


def test_qproj_width_and_workspace_size(lib):
    assert K.kvlr_qproj_width(_shape()) == 96
    assert K.kvlr_qproj_width(_shape(key_mode=K.KVLR_KEYS_LATENT, rank_k=64)) == 64
    ws = K.kvlr_workspace_bytes(_shape(), 16, 512)
    # routing scores alone need B * H_kv * max_pages floats
    assert ws >= 16 * 8 * 512 * 4
    assert K.kvlr_workspace_bytes(_shape(), 16, 0) == 0
    assert K.kvlr_workspace_bytes(_shape(head_dim=96), 16, 512) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), K.KVLR_ERR_UNSUPPORTED),
    (dict(rank_v=48), K.KVLR_ERR_UNSUPPORTED),
    (dict(rank_v=128, dtype=K.KVLR_DTYPE_F32), K.KVLR_ERR_UNSUPPORTED),    # full width: bf16 only
    (dict(page_size=128), K.KVLR_ERR_UNSUPPORTED),
    (dict(num_q_heads=48, num_kv_heads=3), K.KVLR_ERR_UNSUPPORTED),   # G = 16
    (dict(num_q_heads=30), K.KVLR_ERR_INVALID_ARGUMENT),              # not a multiple
    (dict(rank_k=256), K.KVLR_ERR_INVALID_ARGUMENT),                  # above head_dim
    (dict(dtype=7), K.KVLR_ERR_INVALID_ARGUMENT),
    (dict(key_mode=3), K.KVLR_ERR_INVALID_ARGUMENT),
    (dict(num_phys_pages=0), K.KVLR_ERR_INVALID_ARGUMENT),
])
def test_bad_shapes_are_rejected(lib, kw, status):
    s = _shape(**kw)
    f = K.make_factors()
    assert lib.kvlr_upproject(ctypes.byref(s), ctypes.byref(f), None, None, 1, None) == status


def test_bad_arguments_are_rejected_before_launch(lib):
    s = _shape()
    c = K.make_cache()
    f = K.make_factors()
    E = K.KVLR_ERR_INVALID_ARGUMENT
    # null pointers
    assert lib.kvlr_route_pages(ctypes.byref(s), ctypes.byref(c), None, None, None, 512, 1, 8, None, 64,
                                None, None, None, None, None, 0, 16, None) == E
    assert lib.kvlr_decode_attn(ctypes.byref(s), ctypes.byref(c), None, None, None, None, 512, None, None,
                                None, 0, 0.1, None, None, None, 0, 16, None) == E
    assert lib.kvlr_append_encode(ctypes.byref(s), ctypes.byref(f), ctypes.byref(c), None, None,
                                  None, None, None, 512, 16, 16, None) == E
    assert lib.kvlr_project_queries(ctypes.byref(s), ctypes.byref(f), None, None, 16, None) == E
    assert lib.kvlr_append_encode_project(ctypes.byref(s), ctypes.byref(f), ctypes.byref(c), None,
                                          None, None, None, None, 512, 16, 16, None, None,
                                          None) == E
    # k_max below the routing bound, or above max pages
    fake = 1 << 20  # aligned non-null placeholder; never dereferenced on these paths
    c2 = K.make_cache(fake, fake, fake)
    assert lib.kvlr_route_pages(ctypes.byref(s), ctypes.byref(c2), fake, fake, fake, 512, 1, 8, None, 63,
                                fake, None, None, None, fake, 1 << 30, 16, None) == E
    assert lib.kvlr_route_pages(ctypes.byref(s), ctypes.byref(c2), fake, fake, fake, 512, 1, 8, None, 513,
                                fake, None, None, None, fake, 1 << 30, 16, None) == E
    # topk fraction with a zero denominator
    assert lib.kvlr_route_pages(ctypes.byref(s), ctypes.byref(c2), fake, fake, fake, 512, 1, 0, None, 64,
                                fake, None, None, None, fake, 1 << 30, 16, None) == E
    # misaligned pointer
    assert lib.kvlr_route_pages(ctypes.byref(s), ctypes.byref(c2), fake + 4, fake, fake, 512, 1, 8, None,
                                64, fake, None, None, None, fake, 1 << 30, 16, None) == E
    # workspace too small
    assert lib.kvlr_route_pages(ctypes.byref(s), ctypes.byref(c2), fake, fake, fake, 512, 1, 8, None, 64,
                                fake, None, None, None, fake, 16, 16, None) == K.KVLR_ERR_WORKSPACE_TOO_SMALL
    assert lib.kvlr_decode_attn(ctypes.byref(s), ctypes.byref(c2), fake, fake, fake, fake, 512, fake, None,
                                None, 64, 0.1, fake, None, fake, 16, 16, None) == K.KVLR_ERR_WORKSPACE_TOO_SMALL
    # counts without a page list
    assert lib.kvlr_decode_attn(ctypes.byref(s), ctypes.byref(c2), fake, fake, fake, fake, 512, None, None,
                                fake, 64, 0.1, fake, None, fake, 1 << 30, 16, None) == E
    # batch above the supported maximum
    assert lib.kvlr_route_pages(ctypes.byref(s), ctypes.byref(c2), fake, fake, fake, 512, 1, 8, None, 64,
                                fake, None, None, None, fake, 1 << 40, 5000, None) == K.KVLR_ERR_UNSUPPORTED
    assert lib.kvlr_append_encode(ctypes.byref(s), ctypes.byref(f), ctypes.byref(c2), fake, fake,
                                  fake, fake, fake, 512, 5000, 16, None) == K.KVLR_ERR_UNSUPPORTED
    # the fused up-projection needs its output and the factors
    assert lib.kvlr_decode_attn_upproject(ctypes.byref(s), ctypes.byref(f), ctypes.byref(c2), fake, fake,
                                          fake, fake, 512, fake, None, None, 64, 0.1, fake, None, None, fake,
                                          1 << 30, 16, None) == E
    assert lib.kvlr_decode_attn_upproject(ctypes.byref(s), None, ctypes.byref(c2), fake, fake, fake,
                                          fake, 512, fake, None, None, 64, 0.1, fake, None, fake, fake,
                                          1 << 30, 16, None) == E
    # non-positive or non-finite softmax scale
    for sc in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.kvlr_decode_attn(ctypes.byref(s), ctypes.byref(c2), fake, fake, fake, fake, 512,
                                    fake, None, None, 64, sc, fake, None, fake, 1 << 30, 16, None) == E
    # routing reads compressed value latents
    assert lib.kvlr_route_pages(ctypes.byref(_shape(rank_v=128)), ctypes.byref(c2), fake, fake, fake,
                                512, 1, 8, None, 64, fake, None, None, None, fake, 1 << 30, 16,
                                None) == K.KVLR_ERR_UNSUPPORTED
    # routing needs the routed (exact-key) cache
    sl = _shape(key_mode=K.KVLR_KEYS_LATENT, rank_k=64)
    assert lib.kvlr_route_pages(ctypes.byref(sl), ctypes.byref(c2), fake, fake, fake, 512, 1, 8, None, 64,
                                fake, None, None, None, fake, 1 << 30, 16, None) == K.KVLR_ERR_UNSUPPORTED
    # per-sequence page budgets: k_max must be positive, arrays aligned
    assert lib.kvlr_route_pages(ctypes.byref(s), ctypes.byref(c2), fake, fake, fake, 512, 1, 8, fake, 0,
                                fake, None, None, None, fake, 1 << 30, 16, None) == E
    assert lib.kvlr_route_pages(ctypes.byref(s), ctypes.byref(c2), fake, fake, fake, 512, 1, 8, fake + 4,
                                64, fake, None, None, None, fake, 1 << 30, 16, None) == E
    # with budgets the fraction is not read (a zero denominator is accepted)
    assert lib.kvlr_route_pages(ctypes.byref(s), ctypes.byref(c2), fake, fake, fake, 512, 1, 0, fake, 64,
                                fake, None, None, None, fake, 16, 16, None) == K.KVLR_ERR_WORKSPACE_TOO_SMALL
    assert lib.kvlr_route_pages(ctypes.byref(s), ctypes.byref(c2), fake, fake, fake, 512, 1, 8, None, 64,
                                fake, None, fake + 4, None, fake, 1 << 30, 16, None) == E
    # physical page ids need the page ids beside them
    assert lib.kvlr_decode_attn(ctypes.byref(s), ctypes.byref(c2), fake, fake, fake, fake, 512, None,
                                fake, None, 64, 0.1, fake, None, fake, 1 << 30, 16, None) == E
    # negative batch / sizes
    assert lib.kvlr_upproject(ctypes.byref(s), ctypes.byref(f), fake, fake, -1, None) == E
    assert lib.kvlr_append_encode(ctypes.byref(s), ctypes.byref(f), ctypes.byref(c2), fake, fake,
                                  fake, fake, fake, 512, 16, -5, None) == E
    assert lib.kvlr_append_encode(ctypes.byref(s), ctypes.byref(f), ctypes.byref(c2), fake, fake,
                                  fake, fake, fake, 0, 16, 16, None) == E


def test_empty_batches_are_no_ops(lib):
    s = _shape()
    c = K.make_cache()
    f = K.make_factors()
    assert lib.kvlr_upproject(ctypes.byref(s), ctypes.byref(f), None, None, 0, None) == 0
    assert lib.kvlr_project_queries(ctypes.byref(s), ctypes.byref(f), None, None, 0, None) == 0
    assert lib.kvlr_append_encode(ctypes.byref(s), ctypes.byref(f), ctypes.byref(c), None, None,
                                  None, None, None, 512, 16, 0, None) == 0
    assert lib.kvlr_append_encode_project(ctypes.byref(s), ctypes.byref(f), ctypes.byref(c), None,
                                          None, None, None, None, 512, 0, 0, None, None, None) == 0
    assert lib.kvlr_workspace_init(None, 0, None) == 0


def test_python_binding_raises(lib):
    with pytest.raises(K.KvlrError) as ei:
        K.kvlr_upproject(_shape(head_dim=96), K.make_factors(), None, None, 1)
    assert ei.value.status == K.KVLR_ERR_UNSUPPORTED


def test_output_projection_arguments(lib):
    s = _shape()
    f = K.make_factors()
    fake = 1 << 20
    E = K.KVLR_ERR_INVALID_ARGUMENT
    assert lib.kvlr_fold_output_weights(ctypes.byref(s), ctypes.byref(f), fake, 4096, fake, None) == E
    f2 = K.make_factors(B_v=fake)
    assert lib.kvlr_fold_output_weights(ctypes.byref(s), ctypes.byref(f2), fake, 4090, fake, None) == E
    assert lib.kvlr_fold_output_weights(ctypes.byref(s), ctypes.byref(f2), None, 4096, fake, None) == E
    assert lib.kvlr_output_projection(ctypes.byref(s), fake, fake, 4096, fake, -1, None) == E
    assert lib.kvlr_output_projection(ctypes.byref(s), fake, fake, 0, fake, 4, None) == E
    assert lib.kvlr_output_projection(ctypes.byref(s), fake, fake, 4096, fake, 0, None) == 0
    sf = _shape(dtype=K.KVLR_DTYPE_F32)
    assert lib.kvlr_output_projection(ctypes.byref(sf), fake, fake, 4096, fake, 4, None) == \
        K.KVLR_ERR_UNSUPPORTED


def test_fit_arguments(lib):
    s = _shape()
    fake = 1 << 20
    E = K.KVLR_ERR_INVALID_ARGUMENT
    ws = K.kvlr_fit_workspace_bytes(s, 524288)
    # float64 moments plus float32 per-run partials (256 workgroups over 8 heads: 32 runs)
    assert ws >= 8 * 3 * 128 * 128 * (8 + 4 * 32)
    assert K.kvlr_fit_workspace_bytes(s, 0) == 8 * 3 * 128 * 128 * 8
    assert K.kvlr_fit_workspace_bytes(s, -1) == 0
    assert K.kvlr_fit_workspace_bytes(_shape(head_dim=96), 100) == 0
    assert K.kvlr_fit_workspace_bytes(s, 100) < K.kvlr_fit_workspace_bytes(s, 100000)
    mom = lib.kvlr_fit_moments
    assert mom(ctypes.byref(s), fake, fake, 100, fake, 2, fake, ws, None) == E       # accumulate flag
    assert mom(ctypes.byref(s), fake, fake, -1, fake, 0, fake, ws, None) == E
    assert mom(ctypes.byref(s), fake, fake, 100, None, 0, fake, ws, None) == E
    assert mom(ctypes.byref(s), fake + 8, fake, 100, fake, 0, fake, ws, None) == E   # misaligned
    assert mom(ctypes.byref(s), fake, fake, 100000, fake, 0, fake, 1024, None) == \
        K.KVLR_ERR_WORKSPACE_TOO_SMALL
    out = K.make_factor_buffers(fake, fake, fake, fake, None)  # exact keys need W_pred
    fit = lib.kvlr_fit_factors
    assert fit(ctypes.byref(s), fake, fake, 100, ctypes.byref(out), None, None, fake, ws, None) == E
    out = K.make_factor_buffers(fake, fake, fake, fake, fake)
    assert fit(ctypes.byref(s), fake, fake, 0, ctypes.byref(out), None, None, fake, ws, None) == E
    assert fit(ctypes.byref(s), fake, fake, 100000, ctypes.byref(out), None, None, fake, 64,
               None) == K.KVLR_ERR_WORKSPACE_TOO_SMALL
    assert fit(ctypes.byref(_shape(head_dim=96)), fake, fake, 100, ctypes.byref(out), None, None,
               fake, ws, None) == K.KVLR_ERR_UNSUPPORTED
    assert lib.kvlr_fit_solve(ctypes.byref(s), None, fake, fake, fake, None, None) == E
    assert "linear algebra" in K.kvlr_status_string(K.KVLR_ERR_NUMERICAL)
    with pytest.raises(TypeError):
        K.kvlr_fit_solve(s, np.zeros((8, 3, 128, 128), np.float32), np.zeros((8, 128, 64)),
                         np.zeros((8, 128, 32)), np.zeros((8, 64, 128)))


def test_fp8_latent_shapes(lib):
    s = _shape(dtype=K.KVLR_DTYPE_BF16_FP8)
    assert K.kvlr_qproj_width(s) == 96
    assert K.kvlr_workspace_bytes(s, 16, 512) > 0
    U = K.KVLR_ERR_UNSUPPORTED
    f = K.make_factors()
    for bad in (_shape(dtype=K.KVLR_DTYPE_BF16_FP8, page_size=16),
                _shape(dtype=K.KVLR_DTYPE_BF16_FP8, rank_v=128)):
        assert lib.kvlr_upproject(ctypes.byref(bad), ctypes.byref(f), None, None, 1, None) == U
    assert lib.kvlr_upproject(ctypes.byref(_shape(dtype=3)), ctypes.byref(f), None, None, 1,
                              None) == K.KVLR_ERR_INVALID_ARGUMENT


def test_per_head_residual_rank_arguments(lib):
    fake = 1 << 20
    ws = 1 << 40  # size checks pass; nothing below reaches a launch
    f = K.make_factors(fake, fake, fake, fake, fake)

    def route(shape, ranks):
        c = K.make_cache(fake, fake, fake, ranks)
        return lib.kvlr_route_pages(ctypes.byref(shape), ctypes.byref(c), fake, fake, fake, 512, 1, 8, None,
                                    64, fake, None, None, None, fake, ws, 4, None)

    def encode(shape, ranks):
        c = K.make_cache(fake, fake, fake, ranks)
        return lib.kvlr_append_encode(ctypes.byref(shape), ctypes.byref(f), ctypes.byref(c), fake, fake,
                                      fake, fake, fake, 512, 4, 4, None)

    U, E = K.KVLR_ERR_UNSUPPORTED, K.KVLR_ERR_INVALID_ARGUMENT
    s = _shape(rank_k=64)
    for call in (route, encode):
        assert call(s, [16, 32, 64, 48, 16, 16, 16, 16]) == E      # 48 is not a chunk-tile rank
        assert call(_shape(rank_k=32), [64] * 8) == E                # above rank_k
        assert call(_shape(rank_k=64, page_size=32), [16] * 8) == U  # 64-token pages only
        assert call(_shape(rank_k=64, dtype=K.KVLR_DTYPE_F32), [16] * 8) == U
        assert call(_shape(rank_k=64, num_q_heads=68, num_kv_heads=17), [16] * 17) == U  # > 16 heads
    assert encode(_shape(rank_k=64, key_mode=K.KVLR_KEYS_LATENT), [16] * 8) == U   # routed keys only


def test_noalloc_attention_arguments(lib):
    """The allocation-free attention call checks its arguments like the
    workspace one and rejects, before any launch, a call whose chunk records
    would not fit the static scratch."""
    fake = 1 << 20
    s = _shape(key_mode=K.KVLR_KEYS_LATENT, rank_k=64)
    c = K.make_cache(fake, fake, fake)
    f = K.make_factors(fake, fake, fake, fake, fake)
    assert K.kvlr_noalloc_scratch_bytes() == 32 << 20
    # dense attention over 2048 sequences of 65536 pages: 2048 * 8 pairs x 512
    # chunks x 4 heads x 66 floats of chunk records, far above 32 MiB
    assert lib.kvlr_decode_attn_upproject_noalloc(
        ctypes.byref(s), ctypes.byref(f), ctypes.byref(c), fake, fake, fake, fake, 65536, None,
        None, None, 0, 0.1, fake, None, fake, 2048, None) == K.KVLR_ERR_WORKSPACE_TOO_SMALL
    # the output is required, as for kvlr_decode_attn_upproject
    assert lib.kvlr_decode_attn_upproject_noalloc(
        ctypes.byref(s), ctypes.byref(f), ctypes.byref(c), fake, fake, fake, fake, 512, None,
        None, None, 0, 0.1, fake, None, None, 16, None) == K.KVLR_ERR_INVALID_ARGUMENT
    # non-finite scale
    assert lib.kvlr_decode_attn_upproject_noalloc(
        ctypes.byref(s), ctypes.byref(f), ctypes.byref(c), fake, fake, fake, fake, 512, None,
        None, None, 0, float("nan"), fake, None, fake, 16, None) == K.KVLR_ERR_INVALID_ARGUMENT


def test_residual_prep_arguments(lib):
    """Sizes of the prepared residual operand, and the host-side rejections of
    kvlr_prepare_residual and of a misaligned operand handed to the encode."""
    # bf16: ceil(r_v/32) k-steps x r_k/16 tiles x 64 lanes x 8 elements x 2 B, high and low parts
    assert K.kvlr_residual_prep_bytes(_shape()) == 8 * (2 * 2 * 64 * 8 * 2 * 2)
    assert K.kvlr_residual_prep_bytes(_shape(dtype=K.KVLR_DTYPE_BF16_FP8)) == 8 * 8192
    assert K.kvlr_residual_prep_bytes(_shape(head_dim=64, rank_v=32, rank_k=16, num_q_heads=16,
                                             num_kv_heads=2)) == 2 * (1 * 1 * 64 * 8 * 2 * 2)
    # f32: r_v/4 k-steps x r_k/16 tiles x 64 lanes x 4 B, one part
    assert K.kvlr_residual_prep_bytes(_shape(dtype=K.KVLR_DTYPE_F32)) == 8 * (16 * 2 * 64 * 4)
    assert K.kvlr_residual_prep_bytes(_shape(key_mode=K.KVLR_KEYS_LATENT, rank_k=64)) == 0
    assert K.kvlr_residual_prep_bytes(_shape(head_dim=96)) == 0
    fake = 1 << 20
    f = K.make_factors(fake, fake, fake, fake, fake)
    s = _shape()
    need = K.kvlr_residual_prep_bytes(s)

    def prep(shape, factors, ptr, nbytes):
        return lib.kvlr_prepare_residual(ctypes.byref(shape), ctypes.byref(factors), ptr, nbytes, None)

    assert prep(s, f, fake, need - 16) == K.KVLR_ERR_WORKSPACE_TOO_SMALL
    assert prep(s, f, fake + 8, need) == K.KVLR_ERR_INVALID_ARGUMENT
    assert prep(s, f, None, need) == K.KVLR_ERR_INVALID_ARGUMENT
    assert prep(s, K.make_factors(fake, fake, fake, fake, None), fake, need) == K.KVLR_ERR_INVALID_ARGUMENT
    assert prep(_shape(key_mode=K.KVLR_KEYS_LATENT, rank_k=64), f, fake, need) == \
        K.KVLR_ERR_INVALID_ARGUMENT
    with pytest.raises(K.KvlrError):
        K.kvlr_prepare_residual(s, f, None, need)
    # a misaligned operand is rejected by the encode before its launch
    c = K.make_cache(fake, fake, fake)
    fm = K.make_factors(fake, fake, fake, fake, fake, fake + 8)
    assert lib.kvlr_append_encode(ctypes.byref(s), ctypes.byref(fm), ctypes.byref(c), fake, fake,
                                  fake, fake, fake, 512, 4, 4, None) == K.KVLR_ERR_INVALID_ARGUMENT


def test_page_table_check_arguments(lib):
    """kvlr_check_page_tables rejects bad arguments before any launch."""
    fake = 1 << 20
    s = _shape()

    def call(shape, sl, pt, mp, b, err):
        return lib.kvlr_check_page_tables(ctypes.byref(shape), sl, pt, mp, b, err, None)

    assert call(s, fake, fake, 512, 4, None) == K.KVLR_ERR_INVALID_ARGUMENT      # no error words
    assert call(s, fake, fake, 512, 4, fake + 4) == K.KVLR_ERR_INVALID_ARGUMENT  # misaligned
    assert call(s, None, fake, 512, 4, fake) == K.KVLR_ERR_INVALID_ARGUMENT
    assert call(s, fake, fake, 0, 4, fake) == K.KVLR_ERR_INVALID_ARGUMENT
    assert call(s, fake, fake, 512, -1, fake) == K.KVLR_ERR_INVALID_ARGUMENT
    assert call(_shape(head_dim=96), fake, fake, 512, 4, fake) == K.KVLR_ERR_UNSUPPORTED
    assert (K.KVLR_TABLE_ERR_PAGE, K.KVLR_TABLE_ERR_LENGTH) == (1, 2)


def test_score_and_select_arguments(lib):
    """kvlr_score_pages and kvlr_select_pages, the two halves of routing,
    reject bad arguments before any launch."""
    fake = 1 << 20
    s = _shape()
    c = K.make_cache(fake, fake, fake)
    E = K.KVLR_ERR_INVALID_ARGUMENT

    def score(shape, cache, qp, sl, pt, mp, ps, b):
        return lib.kvlr_score_pages(ctypes.byref(shape), ctypes.byref(cache), qp, sl, pt, mp, ps, b, None)

    assert score(s, c, fake, fake, fake, 512, None, 16) == E              # scores are the output
    assert score(s, c, fake, fake, fake, 512, fake + 4, 16) == E          # misaligned
    assert score(s, c, None, fake, fake, 512, fake, 16) == E              # no query images
    assert score(s, c, fake, fake, fake, 0, fake, 16) == E                # empty table rows
    assert score(s, c, fake, fake, fake, 512, fake, 5000) == K.KVLR_ERR_UNSUPPORTED
    assert score(s, c, fake, fake, fake, 512, fake, 0) == K.KVLR_OK       # empty batch: no-op
    assert score(_shape(key_mode=K.KVLR_KEYS_LATENT), c, fake, fake, fake, 512, fake, 16) == \
        K.KVLR_ERR_UNSUPPORTED                                           # routing needs exact keys

    def select(shape, sl, pt, mp, ps, num, den, kp, kmax, sel, cnt, ph, b):
        return lib.kvlr_select_pages(ctypes.byref(shape), sl, pt, mp, ps, num, den, kp, kmax, sel, cnt,
                                     ph, b, None)

    assert select(s, fake, fake, 512, fake, 1, 8, None, 63, fake, None, None, 16) == E   # k_max below bound
    assert select(s, fake, fake, 512, fake, 1, 8, None, 513, fake, None, None, 16) == E  # above the table
    assert select(s, fake, fake, 512, fake, 1, 0, None, 64, fake, None, None, 16) == E   # zero denominator
    assert select(s, fake, fake, 512, None, 1, 8, None, 64, fake, None, None, 16) == E   # no scores
    assert select(s, fake, fake, 512, fake, 1, 8, None, 64, None, None, None, 16) == E   # no page list
    assert select(s, fake, fake, 512, fake, 1, 8, None, 64, fake, fake + 4, None, 16) == E
    assert select(s, fake, fake, 512, fake, 1, 8, fake, 0, fake, None, None, 16) == E    # budgets, k_max 0
    assert select(s, fake, fake, 512, fake, 1, 8, None, 64, fake, None, None, 5000) == K.KVLR_ERR_UNSUPPORTED
    assert select(s, fake, fake, 512, fake, 1, 8, None, 64, fake, None, None, 0) == K.KVLR_OK
