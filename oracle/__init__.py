"""Plain CPU oracle for one decode step of attention over a low-rank
compressed, paged KV cache (BasisKV form).

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package. The HIP library and its Python
binding never import or call it, and it imports nothing from them.
"""

from .kvlr_oracle import (  # noqa: F401
    STORAGE_TYPES,
    round_bf16,
    round_fp8_e4m3,
    round_to_storage,
    encode_tokens,
    append_tokens,
    empty_state,
    project_queries,
    key_approximation,
    page_scores,
    pages_to_keep,
    select_top_pages,
    tokens_of_pages,
    attend,
    upproject,
    decode_pair,
    attend_selected,
    output_projection,
    fold_output_weights,
    latent_output_projection,
    fit_factors,
    choose_residual_ranks,
    latent_outputs,
    staged_decoder,
    fit_joint_decoder,
    fit_partition_decoders,
    fold_decoder,
    complete_output_error,
)
