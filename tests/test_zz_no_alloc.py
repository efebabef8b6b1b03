"""The allocation-free attention entry point against the workspace one.

kvlr_decode_attn_upproject_noalloc runs the same kernels as
kvlr_decode_attn_upproject with the chunk records in the library's static
device scratch instead of a caller workspace, so z, lse and o must be
identical bit for bit. Two calls in a row, the second on a smaller input,
check that the shared scratch carries nothing from one call to the next.
(A call needing more scratch than the array holds is rejected on the host
before launch: tests/test_abi.py.)
"""

import pytest
import torch

from decode_attention_rank_amd import _lib as K
from decode_attention_rank_amd.session import DecodeSession
from decode_attention_rank_amd.workloads import Workload

pytestmark = pytest.mark.gpu


def _wl(B, G, rv, rk, d=128, P=64, routed=True, storage="bf16", seed=21):
    return Workload(name=f"noalloc-B{B}-G{G}", batch=B, num_q_heads=2 * G, num_kv_heads=2,
                    head_dim=d, page_size=P, rank_v=rv, rank_k=rk, storage=storage,
                    key_mode="exact" if routed else "latent", context=0, topk_num=1, topk_den=8,
                    signal_rank=48, shared_rank=min(rv, 16) if routed else 0, noise_std=0.05,
                    seed=seed)


def _noalloc(s, sel=True):
    use_sel = s.sel if (s.wl.routed and sel) else None
    out = {n: torch.full_like(getattr(s, n), float("nan")) for n in ("z", "lse", "o")}
    K.kvlr_decode_attn_upproject_noalloc(
        s.shape, s.kfactors, s.kcache, s.q, s.q_proj, s.seq_lens_dev, s.page_table, s.max_pages,
        use_sel, s.sel_phys if use_sel is not None else None,
        s.sel_counts if (use_sel is not None and s.use_counts) else None,
        s.k_max if use_sel is not None else 0, s.scale, out["z"], out["lse"], out["o"], s.wl.batch)
    return out


def _case(wl, lens):
    print("case noalloc", wl.name, lens, flush=True)
    s = DecodeSession(wl, "cuda", seq_lens=lens, append_per_seq=9)
    s.step()  # encode, route, attention with the workspace
    torch.cuda.synchronize()
    got = _noalloc(s)
    torch.cuda.synchronize()
    for n in ("z", "lse", "o"):
        assert torch.equal(got[n], getattr(s, n)), n
    return s


def test_noalloc_matches_workspace_entry_point_twice():
    assert K.kvlr_noalloc_scratch_bytes() == 32 << 20
    _case(_wl(6, 4, 64, 32), [3000, 4100, 64, 1, 2500, 4096])
    _case(_wl(2, 8, 32, 32), [700, 1500])  # smaller, after the larger call


def test_noalloc_dense_and_small_pages():
    _case(_wl(3, 4, 64, 64, routed=False), [1000, 2049, 5])
    _case(_wl(2, 2, 32, 16, d=64, P=16, storage="f32"), [777, 33])
