"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the same library calls on the same buffers, replayed as one
HIP graph).

The GPU runs the whole step for every (sequence, KV head). For routed
workloads the page set and the page scores of EVERY pair are checked against
the oracle's scores of the same cache (bit-exact outside the tie band: a
dropped page in a long context would hide inside the output tolerance, so the
page set is the guard); the outputs z, o and lse are checked on a sample of
pairs: the first and last pairs, a middle one, and for ragged contexts the
longest and shortest sequences.
"""

import numpy as np
import pytest
import torch

from decode_attention_rank_amd import synth
from decode_attention_rank_amd.session import DecodeSession
from decode_attention_rank_amd.workloads import WORKLOADS
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

FULL = ["llama3-8b-dense-32k", "llama3-8b-routed-32k", "llama3-70b-share-routed-128k",
        "mixed-append-routed-ragged", "llama3-8b-uncompressed-32k", "llama3-8b-routed-fp8-32k",
        "llama3-70b-share-routed-fp8-128k", "llama3-8b-routed-adaptive-32k"]


def _sample(sess):
    wl = sess.wl
    B, Hkv = wl.batch, wl.num_kv_heads
    pairs = [(0, 0), (B - 1, Hkv - 1), (B // 2, Hkv // 2)]
    if wl.ragged:
        L = sess.seq_lens
        pairs += [(int(np.argmax(L)), 1 % Hkv), (int(np.argmin(L)), (Hkv - 1) // 2)]
    seen, out = set(), []
    for p in pairs:
        if p not in seen:
            seen.add(p)
            out.append(p)
    return out


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(name):
    wl = WORKLOADS[name]
    print("case", name, flush=True)
    sess = DecodeSession(wl, "cuda")
    graph = sess.capture()
    graph.replay()
    torch.cuda.synchronize()
    if wl.routed:
        # every pair's page set, end to end (GPU encode of the new tokens)
        sel = sess.sel.cpu().numpy()
        scores = sess.page_scores.cpu().numpy().astype(np.float64)
        bands = 0
        for b in range(wl.batch):
            for g, st in enumerate(H.oracle_states(sess, b)):
                slack = H.new_token_slack(sess, b, g, st)
                bands += H.check_selection(sess, b, g, st, slack, gpu_sel=sel[b, g],
                                           gpu_scores=scores[b, g])
        print(f"  all {wl.batch * wl.num_kv_heads} page sets accepted; "
              f"{bands} pages in tie bands", flush=True)
    pairs = _sample(sess)
    states = {}
    for b, g in pairs:
        H.check_encode(sess, b, g)
        st = H.oracle_state(sess, b, g)
        states[(b, g)] = st
        info = H.check_pair(sess, b, g, state=st, slack=H.new_token_slack(sess, b, g, st))
        print("  end-to-end", (b, g), info, flush=True)
    staged = {b: H.stage_oracle_sequence(sess, b) for b in sorted({b for b, _ in pairs})}
    sess.decode()
    torch.cuda.synchronize()
    for b, g in pairs:
        info = H.check_pair(sess, b, g, state=staged[b][g])
        print("  staged", (b, g), info, flush=True)
    if wl.planted_frac > 0:
        # the planted pages carry a clear routing signal: routing must find them
        for b, g in pairs:
            N = -(-sess.seq_lens[b] // wl.page_size)
            planted = set(synth.planted_pages(wl, b, N).tolist())
            sel = set(sess.sel[b, g].cpu().numpy().tolist())
            recall = len(planted & sel) / len(planted)
            print("  planted recall", (b, g), recall, flush=True)
            assert recall >= 0.9
