"""Named decode workloads: shapes, ranks, routing fraction and the recipe
knobs of their seeded synthetic inputs.

Shapes follow Llama-class decode: head_dim 128, grouped-query attention, 64-
token pages. Nothing here computes anything.
"""

from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    rank_v: int
    rank_k: int
    storage: str            # "bf16" or "f32": latents, factors, keys, values
    key_mode: str           # "latent" (dense low-rank keys) or "exact" (routed)
    context: int            # tokens per sequence after the step's append (fixed lengths)
    topk_num: int = 1       # routed: keep ceil(N * num / den) pages
    topk_den: int = 1
    signal_rank: int = 48   # rank of the synthetic K/V signal
    shared_rank: int = 0    # key coefficients that the V latent carries (routed)
    noise_std: float = 0.05
    planted_frac: float = 0.0   # fraction of pages whose keys lean toward the query
    planted_boost: float = 0.0  # shift, in coefficient standard deviations
    append_per_seq: int = 1     # tokens each sequence appends in one step
    ragged: bool = False        # lognormal per-sequence contexts
    route: bool = True          # exact keys: route (True) or attend every page (False)
    value_basis: str = "random"  # "identity": the value latent is the value itself
    hidden: int = 0             # output features of W_o (0: num_q_heads * head_dim)
    latent_storage: str = ""    # "fp8": latents as OCP FP8 E4M3 (else as `storage`)
    residual_ranks: tuple = ()  # per-KV-head residual ranks (routed; () = rank_k for all)
    ctx_min: int = 0
    ctx_max: int = 0
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def exact(self) -> bool:
        """Original keys are kept (and attention scores them exactly)."""
        return self.key_mode == "exact"

    @property
    def routed(self) -> bool:
        return self.exact and self.route

    def k_rank(self, g: int) -> int:
        """Residual (or key-latent) rank kept for KV head g."""
        return self.residual_ranks[g] if self.residual_ranks else self.rank_k

    @property
    def lat_storage(self) -> str:
        """Storage type of the latents (v_lat, k_lat)."""
        return self.latent_storage or self.storage

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # Tiny multi-head case, float32 storage, every page attended.
    "tiny-dense-mha-512": Workload(
        name="tiny-dense-mha-512", batch=1, num_q_heads=4, num_kv_heads=4,
        head_dim=64, page_size=16, rank_v=16, rank_k=16, storage="f32",
        key_mode="latent", context=512, signal_rank=16, noise_std=0.01, seed=0),
    # Llama-3-8B-shaped decode, dense low-rank keys and values.
    "llama3-8b-dense-32k": Workload(
        name="llama3-8b-dense-32k", batch=16, num_q_heads=32, num_kv_heads=8,
        head_dim=128, page_size=64, rank_v=64, rank_k=64, storage="bf16",
        key_mode="latent", context=32768, signal_rank=48, noise_std=0.05, seed=1),
    # Same shapes, routed: V-latent key prediction + rank-32 key residual,
    # top 1/8 of pages, exact keys on the chosen pages.
    "llama3-8b-routed-32k": Workload(
        name="llama3-8b-routed-32k", batch=16, num_q_heads=32, num_kv_heads=8,
        head_dim=128, page_size=64, rank_v=64, rank_k=32, storage="bf16",
        key_mode="exact", context=32768, topk_num=1, topk_den=8,
        signal_rank=48, shared_rank=32, noise_std=0.05, seed=2),
    # One GPU's head share of Llama-3-70B under 8-way head partitioning:
    # 8 query heads on 1 KV head, 128k context, top 1/16, 5% of pages planted.
    "llama3-70b-share-routed-128k": Workload(
        name="llama3-70b-share-routed-128k", batch=64, num_q_heads=8, num_kv_heads=1,
        head_dim=128, page_size=64, rank_v=32, rank_k=32, storage="bf16",
        key_mode="exact", context=131072, topk_num=1, topk_den=16,
        signal_rank=48, shared_rank=32, noise_std=0.05,
        planted_frac=0.05, planted_boost=4.0, hidden=8192, seed=3),
    # Mixed: every sequence appends a 4096-token chunk (encoded on append),
    # then one routed decode over ragged lognormal contexts.
    "mixed-append-routed-ragged": Workload(
        name="mixed-append-routed-ragged", batch=32, num_q_heads=32, num_kv_heads=8,
        head_dim=128, page_size=64, rank_v=64, rank_k=32, storage="bf16",
        key_mode="exact", context=0, topk_num=1, topk_den=8,
        signal_rank=48, shared_rank=32, noise_std=0.05, append_per_seq=4096,
        ragged=True, ctx_min=4096, ctx_max=131072, seed=4),
    # Uncompressed reference at the 8B shapes: original keys and full-width
    # values (identity value factors), every page attended.
    "llama3-8b-uncompressed-32k": Workload(
        name="llama3-8b-uncompressed-32k", batch=16, num_q_heads=32, num_kv_heads=8,
        head_dim=128, page_size=64, rank_v=128, rank_k=16, storage="bf16",
        key_mode="exact", context=32768, route=False, value_basis="identity",
        signal_rank=48, shared_rank=16, noise_std=0.05, seed=5),
    # The routed 8B and 70B-share caches with FP8 latents: same seeds, so the
    # same inputs as their bf16 counterparts; keys and factors stay bf16.
    "llama3-8b-routed-fp8-32k": Workload(
        name="llama3-8b-routed-fp8-32k", batch=16, num_q_heads=32, num_kv_heads=8,
        head_dim=128, page_size=64, rank_v=64, rank_k=32, storage="bf16",
        latent_storage="fp8", key_mode="exact", context=32768, topk_num=1, topk_den=8,
        signal_rank=48, shared_rank=32, noise_std=0.05, seed=2),
    # Per-head residual ranks (at most 64) on the 8B routed shapes: mean 28.
    "llama3-8b-routed-adaptive-32k": Workload(
        name="llama3-8b-routed-adaptive-32k", batch=16, num_q_heads=32, num_kv_heads=8,
        head_dim=128, page_size=64, rank_v=64, rank_k=64, storage="bf16",
        key_mode="exact", context=32768, topk_num=1, topk_den=8,
        signal_rank=48, shared_rank=32, noise_std=0.05,
        residual_ranks=(16, 32, 16, 64, 16, 32, 16, 32), seed=2),
    "llama3-70b-share-routed-fp8-128k": Workload(
        name="llama3-70b-share-routed-fp8-128k", batch=64, num_q_heads=8, num_kv_heads=1,
        head_dim=128, page_size=64, rank_v=32, rank_k=32, storage="bf16",
        latent_storage="fp8", key_mode="exact", context=131072, topk_num=1, topk_den=16,
        signal_rank=48, shared_rank=32, noise_std=0.05,
        planted_frac=0.05, planted_boost=4.0, hidden=8192, seed=3),
}

DEFAULT_BENCH_WORKLOAD = "llama3-8b-routed-32k"

# Factor-fit calibration cases (samples, not a decode step).
FIT_WORKLOADS = {
    # Factor-fit calibration at the 8B routed shapes: one sample per cached
    # token (16 sequences x 32768), decaying sample spectra.
    "llama3-8b-fit-512k": Workload(
        name="llama3-8b-fit-512k", batch=16, num_q_heads=32, num_kv_heads=8,
        head_dim=128, page_size=64, rank_v=64, rank_k=32, storage="bf16",
        key_mode="exact", context=32768, shared_rank=32, seed=6),
}
DEFAULT_FIT_WORKLOAD = "llama3-8b-fit-512k"
