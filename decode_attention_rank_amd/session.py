"""Device buffers for one decode step and the calls that run it.

A DecodeSession owns the paged cache, the factors, the per-step inputs and
outputs and the workspace for one workload on one GPU, and runs the step as
the library's calls in order:
  append_encode + project_queries (one launch) -> route_pages (routed only)
  -> decode_attn -> upproject.
It stages seeded synthetic inputs (from `synth`) into device memory; every
step of the method itself runs in the HIP kernels.
"""

from __future__ import annotations

import math

import torch

from . import _lib as K
from . import layout, synth
from .workloads import Workload


def kvlr_dtype(wl: Workload) -> int:
    if wl.lat_storage == "fp8":
        if wl.storage != "bf16":
            raise ValueError("FP8 latents go with bf16 keys and factors")
        return K.KVLR_DTYPE_BF16_FP8
    return K.KVLR_DTYPE_BF16 if wl.storage == "bf16" else K.KVLR_DTYPE_F32


class DecodeSession:
    def __init__(self, wl: Workload, device="cuda", *, seq_lens=None, append_per_seq=None,
                 spare_pages: int = 0, tail_fill: float = 0.0, stage_prefix: bool = True,
                 page_table=None, num_phys=None, k_pages=None, residual_prep: bool = True):
        self.wl = wl
        self.device = torch.device(device)
        self.tail_fill = tail_fill
        self.seq_lens = list(seq_lens) if seq_lens is not None else synth.make_seq_lens(wl)
        B = len(self.seq_lens)
        if B != wl.batch:
            raise ValueError("seq_lens must have one entry per sequence")
        a = wl.append_per_seq if append_per_seq is None else append_per_seq
        self.n_new = [min(a, L) for L in self.seq_lens]
        self.lens_before = [L - n for L, n in zip(self.seq_lens, self.n_new)]
        if page_table is None:
            page_table, num_phys = synth.make_page_table(wl, self.seq_lens, spare_pages)
        self.page_table_cpu = page_table
        self.max_pages = page_table.shape[1]
        self.num_phys = num_phys
        dt = synth.storage_dtype(wl)
        self.dtype = dt
        lt = synth.latent_dtype(wl)
        self.lat_dtype = lt
        self.shape = K.make_shape(
            num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads, head_dim=wl.head_dim,
            page_size=wl.page_size, rank_v=wl.rank_v, rank_k=wl.rank_k, dtype=kvlr_dtype(wl),
            key_mode=K.KVLR_KEYS_EXACT if wl.exact else K.KVLR_KEYS_LATENT,
            num_phys_pages=num_phys)
        dev = self.device
        H, P = wl.num_kv_heads, wl.page_size

        # factors, queries
        self.factors = synth.make_factors(wl, dev)
        self.shape_prep_bytes = K.kvlr_residual_prep_bytes(self.shape)
        self.residual_prep = None
        if residual_prep and self.shape_prep_bytes:
            # the encode's -(W_pred A_k), formed once for these factors
            self.residual_prep = torch.empty(self.shape_prep_bytes, dtype=torch.uint8, device=dev)
            K.kvlr_prepare_residual(self.shape, K.make_factors(**self.factors), self.residual_prep,
                                    self.shape_prep_bytes)
        self.kfactors = K.make_factors(**self.factors, residual_prep=self.residual_prep)
        self.q = synth.make_queries(wl, dev)
        self.Qv, self.Qk = synth.bases(wl)

        # paged cache
        self.v_lat = layout.alloc_pages(num_phys, H, wl.rank_v, P, lt, dev, tail_fill)
        if wl.residual_ranks:
            # per-head residual ranks: one compact run of chunk columns per page,
            # head g's r_g / CH columns after those of heads 0 .. g-1
            ch = layout.chunk_elems(lt)
            self.k_off = [sum(wl.residual_ranks[:g]) // ch for g in range(H)]
            flat = layout.alloc_pages(num_phys, 1, sum(wl.residual_ranks), P, lt, dev, tail_fill)
            self.k_lat = flat[:, 0]
        else:
            self.k_lat = layout.alloc_pages(num_phys, H, wl.rank_k, P, lt, dev, tail_fill)
        self.k_exact = (layout.alloc_pages(num_phys, H, wl.head_dim, P, dt, dev, tail_fill)
                        if wl.exact else None)
        self.kcache = K.make_cache(self.v_lat, self.k_lat, self.k_exact,
                                   wl.residual_ranks if wl.residual_ranks else None)

        # lengths and page table on the device
        self.page_table = page_table.to(dev)
        self.seq_lens_dev = torch.tensor(self.seq_lens, dtype=torch.int32, device=dev)
        self.lens_before_dev = torch.tensor(self.lens_before, dtype=torch.int32, device=dev)
        cu = [0]
        for n in self.n_new:
            cu.append(cu[-1] + n)
        self.cu_new = torch.tensor(cu, dtype=torch.int32, device=dev)
        self.total_new = cu[-1]

        # routing bound and outputs; pages kept: the workload's fraction, or a
        # per-sequence budget (k_pages, one int per sequence)
        B, Hq, d = wl.batch, wl.num_q_heads, wl.head_dim
        self.k_pages_cpu = None if k_pages is None else [int(k) for k in k_pages]
        self.k_pages = (None if k_pages is None else
                        torch.tensor(self.k_pages_cpu, dtype=torch.int32, device=dev))
        if wl.routed and k_pages is not None:
            self.k_max = min(self.max_pages, max([1] + self.k_pages_cpu))
        elif wl.routed:
            bound = -(-(self.max_pages * wl.topk_num) // wl.topk_den)
            self.k_max = min(self.max_pages, max(1, bound))
        else:
            self.k_max = 0
        # attention walks k_max page ids per pair unless the pairs keep
        # different numbers of pages (ragged lengths or budgets): then the
        # per-pair counts bound the rows
        self.use_counts = k_pages is not None or len(set(self.seq_lens)) > 1
        self.qp_width = K.kvlr_qproj_width(self.shape)
        self.q_proj = torch.empty(B, Hq, self.qp_width, dtype=torch.float32, device=dev)
        self.sel = (torch.empty(B, H, self.k_max, dtype=torch.int32, device=dev)
                    if wl.routed else None)
        self.sel_counts = (torch.empty(B, H, dtype=torch.int32, device=dev)
                           if wl.routed else None)
        self.sel_phys = (torch.empty(B, H, self.k_max, dtype=torch.int32, device=dev)
                         if wl.routed else None)
        self.page_scores = (torch.empty(B, H, self.max_pages, dtype=torch.float32, device=dev)
                            if wl.routed else None)
        self.z = torch.empty(B, Hq, wl.rank_v, dtype=torch.float32, device=dev)
        self.lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
        self.o = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
        self.ws_bytes = K.kvlr_workspace_bytes(self.shape, B, self.max_pages)
        self.workspace = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=dev)
        K.kvlr_workspace_init(self.workspace, self.ws_bytes)
        self.scale = 1.0 / math.sqrt(d)

        self.k_new = None
        self.v_new = None
        if stage_prefix:
            self.stage_prefix()
            self.stage_new_tokens()

    # ------------------------------------------------------------------ staging
    def prefix_rows(self, b: int):
        """Seeded pre-existing cache rows of sequence b (device tensors [H, n, R])."""
        return synth.synth_latent_cache(self.wl, b, self.lens_before[b], self.device,
                                        q=self.q.cpu(), Qk=self.Qk)

    def stage_prefix(self):
        for b in range(self.wl.batch):
            rows = self.prefix_rows(b)
            self.write_rows(b, rows)

    def k_lat_head(self, g: int) -> torch.Tensor:
        """Pages of KV head g's residual latents, [num_phys, 1, r_g / CH, P, CH]."""
        if not self.wl.residual_ranks:
            return self.k_lat[:, g:g + 1]
        nch = self.wl.k_rank(g) // layout.chunk_elems(self.lat_dtype)
        return self.k_lat[:, self.k_off[g]:self.k_off[g] + nch].unsqueeze(1)

    def write_rows(self, b: int, rows: dict, tail_fill: float | None = None):
        tail_fill = self.tail_fill if tail_fill is None else tail_fill
        pages = self.page_table_cpu[b]
        layout.pack_sequence(self.v_lat, pages, rows["v"], tail_fill)
        if self.wl.residual_ranks:
            for g in range(self.wl.num_kv_heads):
                r = self.wl.k_rank(g)
                layout.pack_sequence(self.k_lat_head(g), pages, rows["k_lat"][g:g + 1, :, :r], tail_fill)
        else:
            layout.pack_sequence(self.k_lat, pages, rows["k_lat"], tail_fill)
        if self.wl.exact:
            layout.pack_sequence(self.k_exact, pages, rows["k_exact"], tail_fill)

    def read_rows(self, b: int, L: int | None = None, start: int = 0) -> dict:
        L = self.seq_lens[b] if L is None else L
        pages = self.page_table_cpu[b]
        if self.wl.residual_ranks:
            # each head's kept coordinates, zero-padded to rank_k
            heads = []
            for g in range(self.wl.num_kv_heads):
                x = layout.unpack_sequence(self.k_lat_head(g), pages, L, start)
                pad = x.new_zeros((1, x.shape[1], self.wl.rank_k - x.shape[2]))
                heads.append(torch.cat([x, pad], dim=2))
            k_lat = torch.cat(heads, dim=0)
        else:
            k_lat = layout.unpack_sequence(self.k_lat, pages, L, start)
        out = {"v": layout.unpack_sequence(self.v_lat, pages, L, start), "k_lat": k_lat}
        if self.wl.exact:
            out["k_exact"] = layout.unpack_sequence(self.k_exact, pages, L, start)
        return out

    def stage_new_tokens(self):
        Ks, Vs = [], []
        for b in range(self.wl.batch):
            Kb, Vb = synth.synth_raw_tokens(self.wl, b, self.lens_before[b], self.n_new[b],
                                            self.device, q=self.q.cpu(), Qv=self.Qv, Qk=self.Qk)
            Ks.append(Kb)
            Vs.append(Vb)
        self.k_new = torch.cat(Ks).contiguous()
        self.v_new = torch.cat(Vs).contiguous()

    # ------------------------------------------------------------------ the step
    def append(self, stream=None):
        K.kvlr_append_encode(self.shape, self.kfactors, self.kcache, self.k_new, self.v_new,
                             self.cu_new, self.lens_before_dev, self.page_table, self.max_pages,
                             self.wl.batch, self.total_new, stream)

    def project_queries(self, stream=None):
        K.kvlr_project_queries(self.shape, self.kfactors, self.q, self.q_proj, self.wl.batch, stream)

    def route(self, stream=None):
        K.kvlr_route_pages(self.shape, self.kcache, self.q_proj, self.seq_lens_dev, self.page_table,
                           self.max_pages, self.wl.topk_num, self.wl.topk_den, self.k_pages,
                           self.k_max, self.sel, self.sel_counts, self.sel_phys, self.page_scores,
                           self.workspace, self.ws_bytes, self.wl.batch, stream)

    def score(self, stream=None):
        """Page scores alone (kvlr_score_pages)."""
        K.kvlr_score_pages(self.shape, self.kcache, self.q_proj, self.seq_lens_dev, self.page_table,
                           self.max_pages, self.page_scores, self.wl.batch, stream)

    def select(self, stream=None):
        """Top-k selection alone from page_scores (kvlr_select_pages)."""
        K.kvlr_select_pages(self.shape, self.seq_lens_dev, self.page_table, self.max_pages,
                            self.page_scores, self.wl.topk_num, self.wl.topk_den, self.k_pages,
                            self.k_max, self.sel, self.sel_counts, self.sel_phys, self.wl.batch,
                            stream)

    def _attn_sel(self, sel, counts, phys):
        use_sel = self.sel if (self.wl.routed and sel) else None
        if counts is None:
            counts = self.use_counts
        use_counts = self.sel_counts if (use_sel is not None and counts) else None
        use_phys = self.sel_phys if (use_sel is not None and phys) else None
        return use_sel, use_phys, use_counts

    def attend(self, stream=None, sel=True, counts=None, phys=True):
        """Attention over the selected pages (or every page), then the merge
        of the chunk records into z and lse."""
        use_sel, use_phys, use_counts = self._attn_sel(sel, counts, phys)
        K.kvlr_decode_attn(self.shape, self.kcache, self.q, self.q_proj, self.seq_lens_dev,
                           self.page_table, self.max_pages, use_sel, use_phys, use_counts,
                           self.k_max if use_sel is not None else 0, self.scale, self.z, self.lse,
                           self.workspace, self.ws_bytes, self.wl.batch, stream)

    def upproject(self, stream=None):
        K.kvlr_upproject(self.shape, self.kfactors, self.z, self.o, self.wl.batch, stream)

    def append_and_project(self, stream=None):
        K.kvlr_append_encode_project(self.shape, self.kfactors, self.kcache, self.k_new, self.v_new,
                                     self.cu_new, self.lens_before_dev, self.page_table,
                                     self.max_pages, self.wl.batch, self.total_new, self.q,
                                     self.q_proj, stream)

    def prepare(self, stream=None):
        """Append-encode and query projection of one step, in one launch where
        both are needed (they are independent)."""
        if self.needs_qproj:
            self.append_and_project(stream)
        else:
            self.append(stream)

    def attend_upproject(self, stream=None, counts=None, phys=True):
        """Attention with the up-projection applied in its merge launch."""
        use_sel, use_phys, use_counts = self._attn_sel(True, counts, phys)
        K.kvlr_decode_attn_upproject(self.shape, self.kfactors, self.kcache, self.q, self.q_proj,
                                     self.seq_lens_dev, self.page_table, self.max_pages, use_sel,
                                     use_phys, use_counts,
                                     self.k_max if use_sel is not None else 0,
                                     self.scale, self.z, self.lse, self.o, self.workspace,
                                     self.ws_bytes, self.wl.batch, stream)

    def finish(self, stream=None, fused=True):
        """Routing (routed caches), attention and up-projection."""
        if self.wl.routed:
            self.route(stream)
        if fused:
            self.attend_upproject(stream)
        else:
            self.attend(stream)
            self.upproject(stream)

    @property
    def needs_qproj(self) -> bool:
        """Projected queries feed routing and latent-key scoring; exact keys
        attended without routing use the queries as they are."""
        return self.wl.routed or not self.wl.exact

    def decode(self, stream=None):
        if self.needs_qproj:
            self.project_queries(stream)
        self.finish(stream)

    def step(self, stream=None, fused=True):
        self.prepare(stream)
        self.finish(stream, fused=fused)

    def capture(self, fused=True) -> torch.cuda.CUDAGraph:
        """The whole step recorded once as a HIP graph (its four launches,
        no memset or copy nodes: the workspace was cleared by a kernel at
        set-up). graph.replay() re-runs the step on the same buffers; the
        launches' host overhead and the gaps between them go away."""
        side = torch.cuda.Stream()  # default priority
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step(fused=fused)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            self.step(fused=fused)
        torch.cuda.synchronize()
        return graph

    # ------------------------------------------------------------ output side
    def prepare_output_projection(self):
        """Draws W_o and folds it onto the value latents (F = W_o blockdiag(B_v^T))."""
        wl = self.wl
        self.hidden = synth.output_width(wl)
        self.W_o = synth.make_output_weight(wl, self.device)
        self.F = torch.empty(self.hidden, wl.num_q_heads * wl.rank_v, dtype=self.dtype,
                             device=self.device)
        self.out = torch.empty(wl.batch, self.hidden, dtype=torch.float32, device=self.device)
        K.kvlr_fold_output_weights(self.shape, self.kfactors, self.W_o, self.hidden, self.F)

    def output_projection(self, stream=None):
        K.kvlr_output_projection(self.shape, self.F, self.z, self.hidden, self.out, self.wl.batch,
                                 stream)

    # ------------------------------------------------------------------ metrics
    def kv_tokens(self) -> int:
        return sum(self.seq_lens)

    def route_bytes(self) -> int:
        """Algorithmic bytes the routing kernel must read: both latents of every valid token."""
        lb = torch.empty(0, dtype=self.lat_dtype).element_size()
        wl = self.wl
        per_token = sum(wl.rank_v + wl.k_rank(g) for g in range(wl.num_kv_heads))
        return sum(self.seq_lens) * per_token * lb

    def attend_bytes(self) -> int:
        """Algorithmic bytes of attention: keys and value latents of the attended tokens."""
        wl = self.wl
        eb = torch.empty(0, dtype=self.dtype).element_size()
        lb = torch.empty(0, dtype=self.lat_dtype).element_size()
        if not wl.routed:
            key = wl.head_dim * eb if wl.exact else wl.rank_k * lb
            return sum(self.seq_lens) * wl.num_kv_heads * (key + wl.rank_v * lb)
        tot = 0
        P = wl.page_size
        for b, L in enumerate(self.seq_lens):
            N = -(-L // P)
            if self.k_pages_cpu is not None:
                k = min(N, max(self.k_pages_cpu[b], 0))
            else:
                k = 0 if N == 0 else min(N, max(1, -(-(N * wl.topk_num) // wl.topk_den)))
            tot += k * P  # upper bound for a ragged last page; exact when pages are full
        return tot * wl.num_kv_heads * (wl.head_dim * eb + wl.rank_v * lb)

    def append_bytes(self, project: bool = True) -> int:
        """Algorithmic bytes of the append launch: the new keys and values
        read, their latents (and original keys) written, the factors read
        once (A_v, A_k and, with a residual, W_pred A_k); with the query
        projection in the same launch also the queries and [W_pred; B_k]
        read and the query images written."""
        wl = self.wl
        eb = torch.empty(0, dtype=self.dtype).element_size()
        lb = torch.empty(0, dtype=self.lat_dtype).element_size()
        H, d, rv, rk = wl.num_kv_heads, wl.head_dim, wl.rank_v, wl.rank_k
        read = self.total_new * H * 2 * d * eb
        lat = sum(rv + wl.k_rank(g) for g in range(H)) * lb
        write = self.total_new * (lat + H * (d * eb if wl.exact else 0))
        weights = H * (d * rv + d * rk + (rv * rk if wl.exact else 0)) * eb
        total = read + write + weights
        if project:
            width = self.qp_width
            total += wl.batch * wl.num_q_heads * d * 4           # queries
            total += H * width * d * eb                          # [W_pred; B_k]
            total += wl.batch * wl.num_q_heads * width * 4       # query images
        return total
