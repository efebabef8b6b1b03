"""GPU parity of the whole decode step against the oracle, on small shapes
that span several tiles and ragged tails, plus edge cases and invariances.

Every case first runs the step end to end (GPU encode, then GPU decode) and
checks it with the tie band widened by the bound on what one-ulp encode
differences can do to a score; then it overwrites the sequences' pages with the
oracle's own encoded cache and checks the decode strictly (bit-exact page sets
outside the 1e-4 tie band, 5e-3 relative output error).
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from decode_attention_rank_amd import _lib as K
from decode_attention_rank_amd.session import DecodeSession
from decode_attention_rank_amd.workloads import Workload
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def make_wl(*, G, d, rv, rk, P, storage, routed, B=4, Hkv=2, topk=(1, 8), seed=11, planted=0.0,
            exact=None, value_basis="random", latent="", ranks=()):
    exact = routed if exact is None else exact
    rs = min(48, d // 2)
    ns = min(rv, rs // 2, d - rk) if exact else 0
    mode = ("routed" if routed else "exact-all") if exact else "latent"
    return Workload(
        name=f"t-G{G}-d{d}-rv{rv}-rk{rk}-P{P}-{storage}{'-' + latent if latent else ''}-{mode}",
        batch=B, num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=d, page_size=P, rank_v=rv,
        rank_k=rk, storage=storage, key_mode="exact" if exact else "latent", context=0,
        topk_num=topk[0], topk_den=topk[1], signal_rank=rs, shared_rank=ns, noise_std=0.05,
        planted_frac=planted, planted_boost=4.0 if planted else 0.0, seed=seed,
        route=routed, value_basis=value_basis, latent_storage=latent, residual_ranks=tuple(ranks))


def run_and_check(sess, pairs=None, stage=True):
    wl = sess.wl
    sess.step()
    torch.cuda.synchronize()
    pairs = pairs or [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    out = []
    for b, g in pairs:
        H.check_encode(sess, b, g)
        st = H.oracle_state(sess, b, g)
        out.append(H.check_pair(sess, b, g, state=st, slack=H.new_token_slack(sess, b, g, st)))
    if stage:
        states = {b: H.stage_oracle_sequence(sess, b) for b in sorted({b for b, _ in pairs})}
        sess.decode()
        torch.cuda.synchronize()
        for b, g in pairs:
            out.append(H.check_pair(sess, b, g, state=states[b][g]))
    return out


ROUTED = [
    dict(G=4, d=128, rv=64, rk=32, P=64, storage="bf16"),
    dict(G=8, d=128, rv=32, rk=32, P=64, storage="bf16"),
    dict(G=1, d=64, rv=16, rk=16, P=16, storage="bf16"),
    dict(G=2, d=64, rv=32, rk=16, P=32, storage="bf16"),
    dict(G=4, d=64, rv=16, rk=32, P=16, storage="f32"),
    dict(G=8, d=128, rv=64, rk=64, P=32, storage="f32"),
]

DENSE = [
    dict(G=4, d=128, rv=64, rk=64, P=64, storage="bf16"),
    dict(G=1, d=64, rv=16, rk=16, P=16, storage="f32"),
    dict(G=8, d=128, rv=32, rk=16, P=32, storage="bf16"),
    dict(G=2, d=64, rv=64, rk=64, P=64, storage="f32"),
]

LENS = [1, 777, 640, 2049]

# FP8 E4M3 latents (bf16 keys and factors): 64-token pages
FP8_ROUTED = [
    dict(G=4, d=128, rv=64, rk=32),
    dict(G=8, d=128, rv=32, rk=32),
    dict(G=1, d=64, rv=16, rk=16),
    dict(G=2, d=64, rv=64, rk=64),
]
FP8_DENSE = [
    dict(G=4, d=128, rv=64, rk=64),
    dict(G=8, d=64, rv=32, rk=16),
]


@pytest.mark.parametrize("cfg", ROUTED, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_routed_small(cfg):
    wl = make_wl(routed=True, **cfg)
    _say("case", wl.name)
    sess = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=37)
    run_and_check(sess)


@pytest.mark.parametrize("cfg", DENSE, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_dense_small(cfg):
    wl = make_wl(routed=False, **cfg)
    _say("case", wl.name)
    sess = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=37)
    run_and_check(sess)


@pytest.mark.parametrize("cfg", FP8_ROUTED, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_fp8_latents_routed(cfg):
    wl = make_wl(routed=True, P=64, storage="bf16", latent="fp8", **cfg)
    _say("case", wl.name)
    sess = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=37)
    assert sess.v_lat.dtype == torch.float8_e4m3fn
    run_and_check(sess)


@pytest.mark.parametrize("cfg", FP8_DENSE, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_fp8_latents_dense(cfg):
    wl = make_wl(routed=False, P=64, storage="bf16", latent="fp8", **cfg)
    _say("case", wl.name)
    sess = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=37)
    run_and_check(sess)


# per-head residual ranks (adaptive residual), routed, 64-token pages
ADAPTIVE = [
    dict(G=4, d=128, rv=64, rk=64, Hkv=2, ranks=(16, 64), latent=""),
    dict(G=8, d=64, rv=32, rk=32, Hkv=2, ranks=(32, 16), latent="fp8"),
    dict(G=2, d=128, rv=32, rk=64, Hkv=4, ranks=(16, 32, 64, 16), latent=""),
    dict(G=1, d=128, rv=64, rk=64, Hkv=4, ranks=(64, 16, 16, 32), latent="fp8"),
]


@pytest.mark.parametrize("cfg", ADAPTIVE, ids=lambda c: "-".join(
    f"{k}{'_'.join(map(str, v)) if isinstance(v, tuple) else v}" for k, v in c.items()))
def test_per_head_residual_ranks(cfg):
    wl = make_wl(routed=True, P=64, storage="bf16", **cfg)
    _say("case", wl.name, wl.residual_ranks)
    sess = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=37, spare_pages=3,
                         tail_fill=float("nan"))
    assert sess.k_lat.shape[1] == sum(wl.residual_ranks) // 8
    run_and_check(sess)


def test_fp8_latents_nan_tails_and_permuted_pages():
    wl = make_wl(G=4, d=128, rv=64, rk=32, P=64, storage="bf16", routed=True, latent="fp8")
    _say("case fp8 NaN tails")
    sess = DecodeSession(wl, "cuda", seq_lens=[65, 777, 130, 1000], append_per_seq=9,
                         spare_pages=7, tail_fill=float("nan"))
    run_and_check(sess)
    assert torch.isfinite(sess.o).all() and torch.isfinite(sess.z).all()


def test_tiny_workload_all_pairs():
    from decode_attention_rank_amd.workloads import WORKLOADS
    wl = WORKLOADS["tiny-dense-mha-512"]
    _say("case", wl.name)
    sess = DecodeSession(wl, "cuda")
    run_and_check(sess)


@pytest.mark.parametrize("topk", [(1, 1), (1, 10 ** 6), (3, 8)])
def test_routing_fraction_extremes(topk):
    # (1, 1): every page kept, so routed attention is dense exact-key attention
    wl = make_wl(G=4, d=128, rv=64, rk=32, P=64, storage="bf16", routed=True, topk=topk)
    _say("case", wl.name, topk)
    sess = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=5)
    run_and_check(sess)
    if topk == (1, 1):
        for b, L in enumerate(LENS):
            N = -(-L // 64)
            sel = sess.sel[b].cpu().numpy()
            assert (sel[:, :N] == np.arange(N)).all()


def test_empty_sequence_in_batch():
    wl = make_wl(G=4, d=64, rv=32, rk=16, P=16, storage="bf16", routed=True, B=3)
    _say("case empty sequence")
    sess = DecodeSession(wl, "cuda", seq_lens=[0, 100, 65], append_per_seq=3)
    run_and_check(sess)
    assert (sess.sel[0].cpu() == -1).all()
    assert torch.isneginf(sess.lse[0]).all()
    assert (sess.z[0] == 0).all() and (sess.o[0] == 0).all()


def test_maximum_batch():
    """The largest batch the boundary accepts (4096 sequences: per-sequence
    offsets and work lists live in LDS), with short ragged contexts, empty
    ones included. Every pair's page count is checked against its closed
    form; sampled pairs, the first and the last against the oracle."""
    B = 4096
    wl = make_wl(G=1, d=64, rv=16, rk=16, P=16, storage="bf16", routed=True, B=B, Hkv=1,
                 topk=(1, 4))
    rng = np.random.default_rng(21)
    lens = [int(x) for x in rng.integers(0, 120, size=B)]
    lens[0], lens[-1] = 119, 0
    _say("case maximum batch", B)
    sess = DecodeSession(wl, "cuda", seq_lens=lens, append_per_seq=1)
    pairs = [(b, 0) for b in sorted({0, 1, B - 2, *rng.choice(B, 40, replace=False).tolist()})]
    run_and_check(sess, pairs=pairs)
    N = -(-np.array(lens) // 16)
    k = np.where(N > 0, np.minimum(N, np.maximum(1, -(-N // 4))), 0)
    assert (sess.sel_counts.cpu().numpy().reshape(B) == k).all()
    assert (sess.sel[B - 1].cpu() == -1).all()


def test_nan_in_unused_slots_and_pages_is_ignored():
    wl = make_wl(G=4, d=128, rv=64, rk=32, P=64, storage="bf16", routed=True)
    _say("case NaN tails")
    sess = DecodeSession(wl, "cuda", seq_lens=[65, 777, 130, 1000], append_per_seq=9,
                         spare_pages=7, tail_fill=float("nan"))
    run_and_check(sess)
    assert torch.isfinite(sess.o).all() and torch.isfinite(sess.z).all()


def test_page_table_permutation_invariance():
    wl = make_wl(G=8, d=128, rv=32, rk=32, P=64, storage="bf16", routed=True)
    _say("case page-table permutation")
    a = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=11)
    pt = a.page_table_cpu.clone()
    g = torch.Generator().manual_seed(5)
    perm = torch.randperm(a.num_phys, generator=g).to(torch.int32)
    pt2 = torch.where(pt >= 0, perm[pt.clamp(min=0).long()], pt)
    b = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=11, page_table=pt2, num_phys=a.num_phys)
    a.step()
    b.step()
    torch.cuda.synchronize()
    for name in ("sel", "page_scores", "z", "lse", "o"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


def test_step_is_deterministic():
    wl = make_wl(G=4, d=128, rv=64, rk=32, P=64, storage="bf16", routed=True)
    _say("case determinism")
    s = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=37)
    s.step()
    torch.cuda.synchronize()
    first = {n: getattr(s, n).clone() for n in ("sel", "page_scores", "z", "lse", "o", "v_lat", "k_lat")}
    for _ in range(3):
        s.step()
    torch.cuda.synchronize()
    for n, t in first.items():
        assert torch.equal(getattr(s, n), t), n


FUSED_CASES = [
    dict(G=4, d=128, rv=64, rk=32, P=64, storage="bf16", routed=True),
    dict(G=8, d=128, rv=32, rk=32, P=64, storage="bf16", routed=True, latent="fp8"),
    dict(G=2, d=64, rv=32, rk=16, P=16, storage="f32", routed=True),
    dict(G=4, d=64, rv=32, rk=32, P=16, storage="bf16", routed=False, exact=False),
]


@pytest.mark.parametrize("kw", FUSED_CASES, ids=["bf16-routed", "fp8-G8", "f32-P16", "latent-keys"])
def test_append_and_projection_in_one_launch(kw):
    """kvlr_append_encode_project gives exactly the two separate calls'
    outputs (cache pages and query images), and with no new tokens the
    projection alone."""
    wl = make_wl(**kw)
    _say("case append+project", wl.name)
    lens = [300, 1000, 77, 129]
    one = DecodeSession(wl, "cuda", seq_lens=lens, append_per_seq=70)
    two = DecodeSession(wl, "cuda", seq_lens=lens, append_per_seq=70)
    one.append()
    one.project_queries()
    two.append_and_project()
    torch.cuda.synchronize()
    assert torch.equal(one.v_lat, two.v_lat)
    assert torch.equal(one.k_lat, two.k_lat)
    if wl.exact:
        assert torch.equal(one.k_exact, two.k_exact)
    assert torch.equal(one.q_proj, two.q_proj)
    two.q_proj.fill_(float("nan"))
    K.kvlr_append_encode_project(two.shape, two.kfactors, two.kcache, None, None, None, None,
                                 two.page_table, two.max_pages, wl.batch, 0, two.q, two.q_proj)
    torch.cuda.synchronize()
    assert torch.equal(one.q_proj, two.q_proj)


PREP_CASES = [
    dict(G=4, d=128, rv=64, rk=32, P=64, storage="bf16", routed=True),
    dict(G=8, d=128, rv=32, rk=32, P=64, storage="bf16", routed=True, latent="fp8"),
    dict(G=2, d=64, rv=32, rk=16, P=16, storage="f32", routed=True),
    dict(G=4, d=128, rv=64, rk=64, P=64, storage="bf16", routed=True, ranks=(16, 64)),
    dict(G=4, d=128, rv=128, rk=16, P=64, storage="bf16", routed=False, exact=True,
         value_basis="identity"),
]


@pytest.mark.parametrize("kw", PREP_CASES, ids=["bf16", "fp8-G8", "f32-P16", "adaptive", "rv128"])
def test_prepared_residual_equals_per_workgroup(kw):
    """kvlr_prepare_residual's operand gives exactly the cache pages that the
    encode writes when each workgroup forms -(W_pred A_k) itself, through both
    append entry points."""
    wl = make_wl(**kw)
    _say("case prepared residual", wl.name)
    lens = [300, 1000, 77, 129]
    own = DecodeSession(wl, "cuda", seq_lens=lens, append_per_seq=70, residual_prep=False)
    pre = DecodeSession(wl, "cuda", seq_lens=lens, append_per_seq=70)
    assert own.residual_prep is None and pre.residual_prep is not None
    assert pre.residual_prep.numel() == K.kvlr_residual_prep_bytes(pre.shape)
    own.append()
    pre.append()
    torch.cuda.synchronize()
    for n in ("v_lat", "k_lat", "k_exact"):
        assert torch.equal(getattr(own, n), getattr(pre, n)), n
    own.append_and_project()
    pre.append_and_project()
    torch.cuda.synchronize()
    for n in ("v_lat", "k_lat", "k_exact", "q_proj"):
        assert torch.equal(getattr(own, n), getattr(pre, n)), n
    # and the pages still match the oracle's encode
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            H.check_encode(pre, b, g)


def test_page_table_check_finds_bad_entries_and_lengths():
    """kvlr_check_page_tables: clean tables give no error; entries in use
    outside [0, num_phys) are flagged and counted (entries past a sequence's
    pages are not looked at); a length beyond its table row is flagged."""
    wl = make_wl(G=4, d=128, rv=64, rk=32, P=64, storage="bf16", routed=True)
    _say("case page-table check")
    lens = [2112, 777, 640, 100]
    sess = DecodeSession(wl, "cuda", seq_lens=lens, append_per_seq=37)
    err = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    pt = sess.page_table.clone()
    K.kvlr_check_page_tables(sess.shape, sess.seq_lens_dev, pt, sess.max_pages, wl.batch, err)
    torch.cuda.synchronize()
    assert err[:2].tolist() == [0, 0]
    n = [-(-L // wl.page_size) for L in lens]
    pt[1, 3] = sess.num_phys + 5           # in use
    pt[2, n[2] - 1] = -2                   # in use (last page)
    pt[3, n[3]] = sess.num_phys + 9        # past sequence 3's pages: not in use
    K.kvlr_check_page_tables(sess.shape, sess.seq_lens_dev, pt, sess.max_pages, wl.batch, err)
    torch.cuda.synchronize()
    assert err[:2].tolist() == [K.KVLR_TABLE_ERR_PAGE, 2]
    long_lens = sess.seq_lens_dev.clone()
    long_lens[0] = sess.max_pages * wl.page_size + 50
    K.kvlr_check_page_tables(sess.shape, long_lens, sess.page_table, sess.max_pages, wl.batch, err)
    torch.cuda.synchronize()
    assert err[:2].tolist() == [K.KVLR_TABLE_ERR_LENGTH, 0]


def test_lengths_past_the_table_row_are_cut_to_it():
    """A sequence length beyond its page-table row (a caller error) is read as
    the row's whole span: routing and attention then equal, bit for bit, the
    step with the length set to that span, and nothing past the row is read
    or written."""
    wl = make_wl(G=4, d=128, rv=64, rk=32, P=64, storage="bf16", routed=True)
    _say("case length past the table row")
    lens = [2112, 777, 640, 100]   # sequence 0 fills its 33-page row exactly
    sess = DecodeSession(wl, "cuda", seq_lens=lens, append_per_seq=37)
    assert sess.max_pages * wl.page_size == lens[0]
    sess.step()
    sess.decode()
    torch.cuda.synchronize()
    ref = {n: getattr(sess, n).clone() for n in ("sel", "sel_counts", "page_scores", "z", "lse", "o")}
    sess.seq_lens_dev[0] = lens[0] + 50
    sess.decode()
    torch.cuda.synchronize()
    for n, t in ref.items():
        assert torch.equal(getattr(sess, n), t), n


@pytest.mark.parametrize("routed", [True, False])
def test_chunked_append_equals_one_shot(routed):
    wl = make_wl(G=4, d=128, rv=64, rk=32 if routed else 64, P=64, storage="bf16", routed=routed)
    _say("case chunked append", routed)
    lens = [300, 1000, 77, 129]
    one = DecodeSession(wl, "cuda", seq_lens=lens, append_per_seq=70)
    two = DecodeSession(wl, "cuda", seq_lens=lens, append_per_seq=70)
    one.append()
    # the same tokens in two calls: first 29 (or fewer) of each sequence, then the rest
    n1 = [min(29, n) for n in two.n_new]
    cu1, cu2, lb2, k1, v1, k2, v2 = [0], [0], [], [], [], [], []
    off = 0
    for b, n in enumerate(two.n_new):
        k1.append(two.k_new[off:off + n1[b]])
        v1.append(two.v_new[off:off + n1[b]])
        k2.append(two.k_new[off + n1[b]:off + n])
        v2.append(two.v_new[off + n1[b]:off + n])
        cu1.append(cu1[-1] + n1[b])
        cu2.append(cu2[-1] + n - n1[b])
        lb2.append(two.lens_before[b] + n1[b])
        off += n
    dev = "cuda"
    for kk, vv, cu, lb in ((k1, v1, cu1, two.lens_before), (k2, v2, cu2, lb2)):
        kt = torch.cat(kk).contiguous()
        vt = torch.cat(vv).contiguous()
        K.kvlr_append_encode(two.shape, two.kfactors, two.kcache, kt, vt,
                             torch.tensor(cu, dtype=torch.int32, device=dev),
                             torch.tensor(lb, dtype=torch.int32, device=dev), two.page_table,
                             two.max_pages, wl.batch, cu[-1])
    torch.cuda.synchronize()
    assert torch.equal(one.v_lat, two.v_lat)
    assert torch.equal(one.k_lat, two.k_lat)
    if routed:
        assert torch.equal(one.k_exact, two.k_exact)


def test_query_projection_and_upprojection_match_oracle():
    wl = make_wl(G=8, d=128, rv=64, rk=32, P=64, storage="bf16", routed=True)
    _say("case q_proj / upproject")
    s = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=1)
    s.step()
    torch.cuda.synchronize()
    qp = H.f64(s.q_proj)
    z = H.f64(s.z)
    o = H.f64(s.o)
    G = wl.group
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            f = H.factors_np(s, g)
            qh, qt = O.project_queries(H.q_group(s, b, g), f["W_pred"], f["B_k"])
            got = qp[b, g * G:(g + 1) * G]
            assert H.rel_err(got, np.concatenate([qh, qt], axis=1)) < 1e-5
            ref = O.upproject(z[b, g * G:(g + 1) * G], f["B_v"])
            assert H.rel_err(o[b, g * G:(g + 1) * G], ref) < 1e-5


def test_binding_reports_bad_launch_arguments():
    wl = make_wl(G=4, d=128, rv=64, rk=32, P=64, storage="bf16", routed=True)
    s = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=1)
    with pytest.raises(K.KvlrError):
        K.kvlr_route_pages(s.shape, s.kcache, s.q_proj, s.seq_lens_dev, s.page_table, s.max_pages,
                           1, 8, None, s.k_max - 1, s.sel, None, None, None, s.workspace, s.ws_bytes, wl.batch)
    with pytest.raises(K.KvlrError):
        K.kvlr_decode_attn(s.shape, s.kcache, s.q, s.q_proj, s.seq_lens_dev, s.page_table,
                           s.max_pages, s.sel, None, None, s.k_max, 0.1, s.z, s.lse, s.workspace, 64, wl.batch)


def test_long_sequence_selects_from_global_scores():
    # more than 4096 pages in one sequence: the selection reads its scores from
    # global memory instead of staging them
    wl = make_wl(G=1, d=64, rv=16, rk=16, P=16, storage="bf16", routed=True, B=2, Hkv=1,
                 topk=(1, 16))
    _say("case long sequence", wl.name)
    sess = DecodeSession(wl, "cuda", seq_lens=[70001, 300], append_per_seq=3)
    out = run_and_check(sess, pairs=[(0, 0), (1, 0)])
    assert -(-70001 // 16) > 4096
    assert all(o.get("tie_band", 0) < 50 for o in out)


def test_exact_ties_go_to_the_lowest_pages():
    # zero queries make every page score exactly 0: the k lowest page indices win
    wl = make_wl(G=4, d=128, rv=64, rk=32, P=64, storage="bf16", routed=True, topk=(3, 8))
    _say("case exact ties")
    sess = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=5)
    sess.q.zero_()
    sess.step()
    torch.cuda.synchronize()
    for b, L in enumerate(LENS):
        N = -(-L // 64)
        k = O.pages_to_keep(N, 3, 8)
        for g in range(wl.num_kv_heads):
            sel = sess.sel[b, g].cpu().numpy()
            assert (sel[:k] == np.arange(k)).all() and (sel[k:] == -1).all()
            assert int(sess.sel_counts[b, g]) == k


@pytest.mark.parametrize("routed", [True, False])
def test_fused_upprojection_matches_separate_calls(routed):
    wl = make_wl(G=8, d=128, rv=32, rk=32 if routed else 16, P=64, storage="bf16", routed=routed)
    _say("case fused up-projection", routed)
    s = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=3)
    s.prepare()
    s.finish(fused=False)
    torch.cuda.synchronize()
    z1, l1, o1 = s.z.clone(), s.lse.clone(), s.o.clone()
    s.o.fill_(float("nan"))
    s.finish(fused=True)
    torch.cuda.synchronize()
    assert torch.equal(s.z, z1) and torch.equal(s.lse, l1)
    assert H.rel_err(H.f64(s.o), H.f64(o1)) < 1e-6


UNCOMPRESSED = [
    dict(G=4, d=128, rv=128, rk=16, P=64),
    dict(G=8, d=128, rv=128, rk=32, P=32),
    dict(G=2, d=64, rv=64, rk=16, P=16),
]


@pytest.mark.parametrize("cfg", UNCOMPRESSED, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_uncompressed_reference(cfg):
    # original keys, values at full width (identity factors), every page attended:
    # plain paged attention, checked against the oracle like the compressed paths
    wl = make_wl(routed=False, exact=True, value_basis="identity", storage="bf16", **cfg)
    _say("case", wl.name)
    sess = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=37)
    run_and_check(sess)
    # the stored value latents are the values themselves
    b = 1
    rows = sess.read_rows(b)
    off = sum(sess.n_new[:b])
    n = sess.n_new[b]
    assert torch.equal(rows["v"][:, sess.lens_before[b]:].cpu(),
                       sess.v_new[off:off + n].transpose(0, 1).cpu())


@pytest.mark.parametrize("cfg", [dict(G=4, d=128, rv=64, rk=32, P=64, B=5),
                                 dict(G=8, d=128, rv=32, rk=32, P=64, B=3),
                                 dict(G=2, d=64, rv=16, rk=16, P=16, B=20, hidden=208)],
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_output_projection_fold(cfg):
    # F = W_o blockdiag(B_v^T) formed on the GPU, then applied to the step's z;
    # checked against the oracle's plain output projection of its own outputs
    # (hidden 208 = 13 output tiles: an odd count for the 32-column tiles)
    cfg = dict(cfg)
    hidden = cfg.pop("hidden", 0)
    wl = make_wl(routed=True, storage="bf16", **cfg).scaled(hidden=hidden)
    _say("case output projection", wl.name)
    lens = [777, 1, 640, 2049, 65] * 4
    s = DecodeSession(wl, "cuda", seq_lens=lens[:wl.batch], append_per_seq=3)
    s.step()
    s.prepare_output_projection()
    s.output_projection()
    torch.cuda.synchronize()
    G, Hq = wl.group, wl.num_q_heads
    Bv = np.stack([H.f64(s.factors["B_v"][h // G]) for h in range(Hq)])
    Wo = H.f64(s.W_o)
    F_ref = O.fold_output_weights(Bv, Wo)
    # F: one bf16 rounding of a float32 sum of exact products, so within one
    # bf16 unit of the exact value plus the float32 accumulation bound
    acc_bound = wl.head_dim * 2.0 ** -24 * O.fold_output_weights(np.abs(Bv), np.abs(Wo))
    Fg = H.f64(s.F)
    assert np.all(np.abs(Fg - F_ref) <= H.bf16_ulp(np.abs(F_ref)) + acc_bound)
    for b in range(wl.batch):
        z = []
        for g in range(wl.num_kv_heads):
            st = H.oracle_state(s, b, g)
            f = H.factors_np(s, g)
            pages = [int(j) for j in s.sel[b, g].cpu().numpy() if j >= 0]
            zz, _, _ = O.attend_selected(H.q_group(s, b, g), st, f, s.seq_lens[b], wl.page_size,
                                         pages, key_mode=wl.key_mode, scale=s.scale)
            z.append(zz)
        z = np.concatenate(z)  # [Hq, r_v]
        o = np.stack([O.upproject(z[h], Bv[h]) for h in range(Hq)])
        ref = O.output_projection(o, Wo)
        assert H.rel_err(H.f64(s.out[b]), ref) <= H.OUT_TOL


GRAPH_CASES = [
    dict(G=4, d=128, rv=64, rk=32, P=64, storage="bf16", routed=True),
    dict(G=8, d=128, rv=32, rk=32, P=64, storage="bf16", routed=True, latent="fp8"),
    dict(G=4, d=128, rv=64, rk=64, P=64, storage="bf16", routed=False),
    dict(G=2, d=64, rv=32, rk=16, P=16, storage="f32", routed=True),
]


@pytest.mark.parametrize("fused", [False, True], ids=["separate-upproject", "fused-upproject"])
@pytest.mark.parametrize("kw", GRAPH_CASES, ids=["bf16-routed", "fp8-G8", "dense", "f32-P16"])
def test_graph_replay_matches_eager(kw, fused):
    """The step captured as a HIP graph: every replay, with the program's own
    eager work (output buffers overwritten, other kernels) and
    synchronisations between replays, gives exactly the eager step's outputs
    and cache pages."""
    wl = make_wl(**kw)
    _say("case graph", wl.name, "fused" if fused else "separate")
    s = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=37)
    s.step(fused=fused)
    torch.cuda.synchronize()
    names = [n for n in ("sel", "sel_counts", "page_scores", "z", "lse", "o", "q_proj", "v_lat",
                         "k_lat", "k_exact") if getattr(s, n, None) is not None]
    ref = {n: getattr(s, n).clone() for n in names}
    g = s.capture(fused=fused)
    for rep in range(4):
        for n in ("z", "lse", "o", "q_proj") + (("sel", "page_scores") if wl.routed else ()):
            getattr(s, n).fill_(-7)
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for n in names:
            assert torch.equal(getattr(s, n), ref[n]), f"replay {rep}: {n} differs from the eager step"
    del g


@pytest.mark.parametrize("kw", [dict(G=4, d=128, rv=64, rk=32, P=64, storage="bf16"),
                                dict(G=8, d=128, rv=32, rk=32, P=64, storage="bf16", latent="fp8"),
                                dict(G=2, d=64, rv=32, rk=16, P=16, storage="f32")],
                         ids=["bf16", "fp8-G8", "f32-P16"])
def test_per_sequence_page_budgets(kw):
    """Routing with a caller-given number of pages per sequence (k_pages):
    each pair keeps min(N_b, k_b) pages, checked against the oracle's scores
    and brute-force top-k rule; zero budgets attend nothing; budgets above
    the page count keep every page."""
    wl = make_wl(routed=True, **kw)
    _say("case k_pages", wl.name)
    sess = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=37, k_pages=[1, 0, 3, 200])
    run_and_check(sess)
    counts = sess.sel_counts.cpu().numpy()
    N = [-(-L // wl.page_size) for L in LENS]
    for b in range(wl.batch):
        assert (counts[b] == min(N[b], [1, 0, 3, 200][b])).all()
    assert torch.all(torch.isneginf(sess.lse[1])) and torch.all(sess.z[1] == 0)


@pytest.mark.parametrize("kw", [dict(G=4, d=128, rv=64, rk=32, P=64, storage="bf16"),
                                dict(G=1, d=64, rv=16, rk=16, P=16, storage="bf16")],
                         ids=["P64", "P16"])
def test_attention_walks_agree(kw):
    """Attention over routed pages gives bit-identical z, lse and o whether
    it walks every pair's k_max page ids (skipping -1 padding) or only the
    counted ones, and whether it addresses pages through the physical ids
    routing wrote or through the page table."""
    wl = make_wl(routed=True, **kw)
    _say("case walks", wl.name)
    s = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=37, k_pages=[1, 0, 3, 7])
    s.prepare()
    s.route()
    outs = []
    for counts, phys in ((True, True), (False, True), (True, False), (False, False)):
        s.attend_upproject(counts=counts, phys=phys)
        torch.cuda.synchronize()
        outs.append({n: getattr(s, n).clone() for n in ("z", "lse", "o")})
    for o in outs[1:]:
        for n in ("z", "lse", "o"):
            assert torch.equal(o[n], outs[0][n]), n


@pytest.mark.parametrize("kw", [dict(G=4, d=128, rv=64, rk=32, P=64, storage="bf16"),
                                dict(G=8, d=128, rv=32, rk=32, P=64, storage="bf16", latent="fp8"),
                                dict(G=2, d=64, rv=32, rk=16, P=32, storage="bf16"),
                                dict(G=4, d=64, rv=16, rk=32, P=16, storage="f32")],
                         ids=["bf16-G4", "fp8-G8", "P32", "f32-P16"])
@pytest.mark.parametrize("budgets", [None, [1, 0, 3, 200]], ids=["fraction", "budgets"])
def test_score_then_select_equals_routing(kw, budgets):
    """kvlr_score_pages writes exactly the page scores kvlr_route_pages
    writes (-inf past each sequence's pages), and kvlr_select_pages after it
    exactly its page sets, physical pages and counts; ragged lengths, the
    fraction and per-sequence budgets (0, 1, 3, more than N)."""
    wl = make_wl(routed=True, **kw)
    _say("case scores then selection", wl.name, budgets)
    s = DecodeSession(wl, "cuda", seq_lens=LENS, append_per_seq=5, k_pages=budgets)
    s.prepare()
    s.route()
    torch.cuda.synchronize()
    names = ("page_scores", "sel", "sel_phys", "sel_counts")
    ref = {n: getattr(s, n).clone() for n in names}
    for n in names:
        getattr(s, n).fill_(-7)
    s.score()
    torch.cuda.synchronize()
    assert torch.equal(s.page_scores, ref["page_scores"])
    s.select()
    torch.cuda.synchronize()
    for n in names:
        assert torch.equal(getattr(s, n), ref[n]), n
