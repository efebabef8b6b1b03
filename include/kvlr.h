/*
 * kvlr -- decode attention read directly from a low-rank compressed, paged
 * KV cache, in the BasisKV form, for AMD Instinct MI355X (gfx950).
 *
 * Source: "BasisKV: Value Latents for Communication and Key Routing"
 * (English abstract; method-details section). Keys and values are compressed
 * by low-rank projections; the value cache keeps rank-r_v latents; the stored
 * value latent predicts part of each key and a key-specific residual latent
 * holds the rest, and together they rank the key pages; the original keys of
 * the chosen pages alone give exact QK scores; the value latent is tied to the
 * output projection, so the up-projection is applied once per head.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a device pointer unless marked "host".
 *     The caller owns every buffer; the library allocates no device memory
 *     and keeps no mutable global state (only the text of each calling
 *     thread's last HIP error, kept per thread), except the static scratch
 *     array of kvlr_decode_attn_upproject_noalloc. Calls are thread-safe;
 *     calls of that entry point must not overlap on one GPU.
 *   - Each call validates its arguments on the host, then enqueues its
 *     kernels on `stream` (a hipStream_t; NULL = the default stream) and
 *     returns without synchronising. Outputs are valid once the stream has
 *     reached the call. A non-zero status means nothing was enqueued, except
 *     KVLR_ERR_HIP, which reports a failed launch. The calibration calls
 *     kvlr_fit_solve and kvlr_fit_factors are the exceptions: they work on
 *     the host (and the latter synchronises), as their comments say.
 *   - Device arrays must be 16-byte aligned. Integer arrays are int32.
 *   - Values that only the device holds (sequence lengths, page tables) are
 *     trusted: the caller keeps every referenced page id inside
 *     [0, num_phys_pages) and every length inside max_pages_per_seq pages.
 *
 * Storage types (kvlr_shape.dtype): KVLR_DTYPE_BF16 or KVLR_DTYPE_F32 for
 * the latents, the original keys, the factors and the new keys/values.
 * KVLR_DTYPE_BF16_FP8 keeps everything bf16 except the latents (v_lat,
 * k_lat), which are stored as OCP 8-bit floats E4M3 (4 exponent bits, bias
 * 7, 3 significand bits, no infinities, largest finite value 448): the
 * append encode rounds each latent once from its float32 value, to nearest
 * even, saturating at +-448 (NaN stays NaN); readers decode exactly. This is
 * a lossy latent codec in the spirit of the page "PackKV: Reducing KV Cache
 * Memory Footprint through LLM-Aware Lossy Compression" (abstract); it halves
 * the bytes that routing and the value side of attention stream. Supported
 * with page_size 64 and rank_v <= 64 only.
 * Queries, projected queries, z, lse and outputs are float32.
 *
 * Cache layout (one "chunk" = CH elements in 16 bytes: 8 bf16 or 4 f32; FP8
 * latents: 8 elements in 8 bytes):
 *   v_lat   [num_phys_pages][H_kv][rank_v  / CH][page_size][CH]
 *   k_lat   [num_phys_pages][H_kv][rank_k  / CH][page_size][CH]
 *   k_exact [num_phys_pages][H_kv][head_dim/ CH][page_size][CH]
 * Token slot s of a page holds, for chunk c, elements c*CH .. c*CH+CH-1 of
 * its row, so the P tokens of one chunk column sit in P*16 (FP8: P*8)
 * contiguous bytes.
 * Logical page j of sequence b (tokens j*P .. j*P+P-1) lives in physical page
 * page_table[b * max_pages_per_seq + j].
 *
 * Factor layouts (per KV head g, row-major):
 *   A_v [H_kv][head_dim][rank_v]    v = V . A_v           (value encode)
 *   B_v [H_kv][rank_v][head_dim]    o = z . B_v           (up-projection)
 *   A_k [H_kv][head_dim][rank_k]    residual / key-latent encode
 *   B_k [H_kv][rank_k][head_dim]    residual / key-latent decode
 *   W_pred [H_kv][rank_v][head_dim] key prediction from the value latent
 *                                   (KVLR_KEYS_EXACT only)
 *
 * Key modes (kvlr_shape.key_mode):
 *   KVLR_KEYS_EXACT  routed BasisKV: k_lat holds the residual latent
 *                    c = (K - v . W_pred) . A_k, k_exact the original keys.
 *   KVLR_KEYS_LATENT dense low-rank keys: k_lat holds k = K . A_k; no
 *                    routing, no original keys.
 *
 * Per-head residual ranks (kvlr_cache.k_lat_ranks != NULL): an adaptive
 * residual in the sense of BasisKV's method details (key design: a residual
 * mechanism that adapts to what the value cannot recover), read as a rank
 * chosen per KV head. KV head g keeps only the first r_g = k_lat_ranks[g]
 * residual coordinates (r_g in {16, 32, 64}, r_g <= rank_k): k_lat becomes
 *   k_lat [num_phys_pages][sum_g r_g / 8][page_size][8 elements]
 * with head g's r_g / 8 chunk columns at chunk offset sum_{g' < g} r_g' / 8.
 * The factors keep their rank_k-wide shapes; residual coordinates at or past
 * r_g are neither stored nor read (their factor columns are ignored), so
 * routing streams (rank_v + r_g) latent elements per token of head g. Needs
 * KVLR_KEYS_EXACT, page_size 64, bf16 or FP8 latents with bf16 factors, and
 * at most 16 KV heads; other shapes return KVLR_ERR_UNSUPPORTED. Only
 * kvlr_append_encode and kvlr_route_pages read the table (attention of a
 * routed cache reads original keys and value latents only).
 *
 * Query-head h belongs to KV head h / G, G = num_q_heads / num_kv_heads.
 * Supported: head_dim in {64, 128}; rank_v, rank_k in {16, 32, 64} and
 * <= head_dim, and rank_v = 128 with bf16 storage (values kept at full
 * width: the uncompressed reference, attended without routing);
 * page_size in {16, 32, 64};
 * G in {1, 2, 4, 8}; max_pages_per_seq <= 65536; batch <= 4096.
 * Other values return KVLR_ERR_UNSUPPORTED.
 */
#ifndef KVLR_H
#define KVLR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvlr_status;
#define KVLR_OK 0
#define KVLR_ERR_INVALID_ARGUMENT 1
#define KVLR_ERR_UNSUPPORTED 2
#define KVLR_ERR_WORKSPACE_TOO_SMALL 3
#define KVLR_ERR_HIP 4
#define KVLR_ERR_NUMERICAL 5   /* factor fit: rank-deficient samples */

#define KVLR_DTYPE_BF16 0
#define KVLR_DTYPE_F32 1
#define KVLR_DTYPE_BF16_FP8 2  /* bf16, except the latents: OCP FP8 E4M3 */

#define KVLR_KEYS_LATENT 0
#define KVLR_KEYS_EXACT 1

typedef struct kvlr_shape {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t rank_v;
  int32_t rank_k;
  int32_t dtype;          /* KVLR_DTYPE_* */
  int32_t key_mode;       /* KVLR_KEYS_* */
  int32_t num_phys_pages;
} kvlr_shape;

typedef struct kvlr_cache {
  void* v_lat;
  void* k_lat;
  void* k_exact;          /* KVLR_KEYS_EXACT only, else NULL */
  const int32_t* k_lat_ranks;  /* host [H_kv] per-head residual ranks, or NULL */
} kvlr_cache;

typedef struct kvlr_factors {
  const void* A_v;
  const void* B_v;
  const void* A_k;
  const void* B_k;
  const void* W_pred;     /* KVLR_KEYS_EXACT only, else NULL */
  /* Optional, KVLR_KEYS_EXACT only: the encode's residual operand written by
   * kvlr_prepare_residual from THESE A_k and W_pred (device, 16-byte
   * aligned), or NULL to have every encode workgroup form it. A stale one
   * (factors changed since) gives wrong residual latents: the caller keeps
   * the two in step. Ignored with KVLR_KEYS_LATENT. */
  const void* residual_prep;
} kvlr_factors;

/*
 * Append-side encode. BasisKV English abstract: new keys and values are
 * compressed on write by the low-rank projections; the residual is what the
 * stored value latent cannot predict of the key.
 *
 * For each new token i of sequence b (cu_new[b] <= i < cu_new[b+1]) and KV
 * head g, at logical position p = seq_lens_before[b] + i - cu_new[b]:
 *   v = RNE(V_i . A_v)
 *   EXACT:  c = RNE((K_i - v . W_pred) . A_k) into k_lat, K_i into k_exact
 *   LATENT: k = RNE(K_i . A_k) into k_lat
 * RNE = round to nearest even in the storage type; arithmetic in float32
 * (bf16 operands on matrix cores, float32 accumulation).
 *   k_new, v_new     [total_new][H_kv][head_dim], storage type
 *   cu_new           [batch + 1] prefix offsets, cu_new[0] = 0,
 *                    cu_new[batch] = total_new
 *   seq_lens_before  [batch]
 *   page_table       [batch][max_pages_per_seq]; pages that the new tokens
 *                    land on must already be mapped
 *   total_new        host; 0 is a no-op
 * Sequence lengths are not updated: the caller owns them.
 */
kvlr_status kvlr_append_encode(const kvlr_shape* shape, const kvlr_factors* factors,
                               const kvlr_cache* cache, const void* k_new, const void* v_new,
                               const int32_t* cu_new, const int32_t* seq_lens_before,
                               const int32_t* page_table, int32_t max_pages_per_seq,
                               int32_t batch, int32_t total_new, void* stream);

/*
 * Query images in latent space (the query side of latent-space scoring).
 * BasisKV English abstract: the value latent stands in for part of the key
 * and the residual latent for the rest, so scores against latents need the
 * query mapped through the same factors.
 *   q       [batch][num_q_heads][head_dim] float32
 *   q_proj  [batch][num_q_heads][kvlr_qproj_width(shape)] float32, out:
 *           EXACT:  [q . W_pred^T (rank_v), q . B_k^T (rank_k)]
 *           LATENT: [q . B_k^T (rank_k)]
 */
kvlr_status kvlr_project_queries(const kvlr_shape* shape, const kvlr_factors* factors,
                                 const float* q, float* q_proj, int32_t batch, void* stream);

/* Floats per (sequence, query head) row of q_proj; 0 for an invalid shape. */
int32_t kvlr_qproj_width(const kvlr_shape* shape);

/*
 * kvlr_append_encode and kvlr_project_queries of one decode step, in one
 * launch. The two are independent (the new tokens' latents and the query
 * images), so the projection's tiles run beside the encode's workgroups
 * instead of in a launch of their own.
 * Arguments as for the two calls; q and q_proj are required, the append's
 * buffers only when total_new > 0 (total_new = 0 runs the projection alone).
 * The outputs are exactly those of the two calls: the same kernels' code
 * computes them. A shape the encode does not support fails as it does there.
 */
kvlr_status kvlr_append_encode_project(const kvlr_shape* shape, const kvlr_factors* factors,
                                       const kvlr_cache* cache, const void* k_new,
                                       const void* v_new, const int32_t* cu_new,
                                       const int32_t* seq_lens_before, const int32_t* page_table,
                                       int32_t max_pages_per_seq, int32_t batch, int32_t total_new,
                                       const float* q, float* q_proj, void* stream);

/*
 * Page routing (KVLR_KEYS_EXACT only). BasisKV English abstract: the value
 * latent's key prediction plus the key-specific residual rank the key pages,
 * and only the chosen pages are read exactly; the abstract leaves the number
 * of pages kept to the caller.
 * For each sequence b and KV head g, with L = seq_lens[b], N = ceil(L / P):
 *   s[h, t] = q_hat_h . v_t + q_tilde_h . c_t    (t < L, h in the group)
 *   S[j]    = max over the group's heads and the valid tokens of page j
 *   k_b     = min(N, k_pages[b]) with a per-sequence budget, else
 *             min(N, max(1, ceil(N * topk_num / topk_den))); 0 if N = 0
 *   sel     = the k_b pages of largest S, equal scores to the lower index,
 *             written in ascending order, then -1 up to k_max
 *   q_proj       from kvlr_project_queries (the routing query images are
 *                made once per step, where the append launch can carry them)
 *   seq_lens     [batch]
 *   page_table   [batch][max_pages_per_seq]
 *   topk_num, topk_den  host; the fraction of pages kept when k_pages is
 *                NULL (ignored otherwise)
 *   k_pages      optional [batch] device budgets, each in [0, k_max]
 *                (values above k_max keep k_max pages, negative ones none)
 *   k_max        host; with k_pages: 1 <= k_max <= max_pages_per_seq; else
 *                at least min(max_pages_per_seq,
 *                ceil(max_pages_per_seq * topk_num / topk_den))
 *   sel_pages    out [batch][H_kv][k_max] logical page ids
 *   sel_counts   optional out [batch][H_kv]: k_b, the number of valid
 *                entries at the front of each sel_pages row
 *   sel_phys     optional out [batch][H_kv][k_max]: page_table entry of each
 *                selected page, -1 beside the -1 padding (lets attention
 *                address the pages without a second lookup)
 *   page_scores  optional out [batch][H_kv][max_pages_per_seq] float32
 *                (S, then -inf past N); NULL keeps them in the workspace
 *   workspace    >= kvlr_workspace_bytes(...) bytes, zero-filled once
 *                before its first use (kvlr_workspace_init); every call
 *                leaves it ready for the next one. Calls sharing one
 *                workspace must not overlap.
 * Scores are unscaled; NaN inputs give an unspecified selection.
 * rank_v above 64 returns KVLR_ERR_UNSUPPORTED.
 * Two launches: the scores (as kvlr_score_pages), then the selection (as
 * kvlr_select_pages, one workgroup per pair).
 */
kvlr_status kvlr_route_pages(const kvlr_shape* shape, const kvlr_cache* cache, const float* q_proj,
                             const int32_t* seq_lens, const int32_t* page_table,
                             int32_t max_pages_per_seq, int32_t topk_num, int32_t topk_den,
                             const int32_t* k_pages, int32_t k_max, int32_t* sel_pages,
                             int32_t* sel_counts, int32_t* sel_phys, float* page_scores,
                             void* workspace, size_t ws_bytes, int32_t batch, void* stream);

/*
 * Page scores alone (KVLR_KEYS_EXACT only): kvlr_route_pages without the
 * selection, for callers that rank or select pages themselves. BasisKV
 * English abstract: the value latent's key prediction plus the key-specific
 * residual score the key pages.
 *   page_scores  out [batch][H_kv][max_pages_per_seq] float32: S[j] as
 *                kvlr_route_pages defines it for j < N, -inf past N
 * Other arguments as for kvlr_route_pages; no workspace is read or written.
 * The scores are exactly those kvlr_route_pages writes (the same kernel).
 * rank_v above 64 returns KVLR_ERR_UNSUPPORTED.
 */
kvlr_status kvlr_score_pages(const kvlr_shape* shape, const kvlr_cache* cache, const float* q_proj,
                             const int32_t* seq_lens, const int32_t* page_table,
                             int32_t max_pages_per_seq, float* page_scores, int32_t batch,
                             void* stream);

/*
 * Top-k page selection alone, from page scores (kvlr_score_pages writes
 * them): the second half of kvlr_route_pages, one workgroup per (sequence,
 * KV head) pair. BasisKV English abstract: the approximate page scores
 * decide which key pages are read; the abstract leaves how many to the
 * caller.
 *   page_scores  [batch][H_kv][max_pages_per_seq] float32, read; entries
 *                past each sequence's N pages are set to -inf
 *   seq_lens, page_table, topk_num, topk_den, k_pages, k_max, sel_pages,
 *   sel_counts, sel_phys   as for kvlr_route_pages (same k_b, order, padding)
 * kvlr_route_pages runs kvlr_score_pages and then this selection; the two
 * calls in a row give exactly its outputs. NaN scores give an unspecified
 * selection.
 */
kvlr_status kvlr_select_pages(const kvlr_shape* shape, const int32_t* seq_lens,
                              const int32_t* page_table, int32_t max_pages_per_seq,
                              float* page_scores, int32_t topk_num, int32_t topk_den,
                              const int32_t* k_pages, int32_t k_max, int32_t* sel_pages,
                              int32_t* sel_counts, int32_t* sel_phys, int32_t batch, void* stream);

/*
 * Decode attention over the compressed cache. BasisKV English abstract:
 * exact QK on the original keys of the chosen pages; the value side stays
 * in latent space, z = sum_t p_t v_t, and B_v is applied afterwards
 * (kvlr_upproject).
 * For each sequence b, query head h (KV head g = h / G), over the tokens t of
 * the attended pages with t < seq_lens[b]:
 *   EXACT:  s_t = scale * q_h . K_t (original keys)
 *   LATENT: s_t = scale * q_tilde_h . k_t (key latents)
 *   p = softmax(s);  z_out[b][h] = sum_t p_t v_t;  lse_out = log sum exp s
 * Attended pages: sel_pages[b][g][0 .. n) with -1 entries skipped, where
 * n = sel_counts[b][g] when sel_counts is given (entries past it are not
 * read) and n = k_max otherwise; or every page 0 .. N-1 when sel_pages is
 * NULL. An empty set gives z = 0 and lse = -inf. Without sel_counts every
 * pair walks k_max entries, which suits batches whose pairs keep about the
 * same number of pages; with it, ragged batches skip their empty rows.
 *   q        [batch][num_q_heads][head_dim] float32 (EXACT; may be NULL in LATENT)
 *   q_proj   from kvlr_project_queries (LATENT; may be NULL in EXACT)
 *   sel_phys optional [batch][H_kv][k_max]: the physical page of each
 *            sel_pages entry (kvlr_route_pages writes it); NULL reads the
 *            page table
 *   z_out    out [batch][num_q_heads][rank_v] float32
 *   lse_out  optional out [batch][num_q_heads] float32 (natural log)
 *   workspace, ws_bytes: as for kvlr_route_pages
 * Two launches: the attention over page chunks, then the merge of each
 * pair's chunk records into z and lse.
 */
kvlr_status kvlr_decode_attn(const kvlr_shape* shape, const kvlr_cache* cache, const float* q,
                             const float* q_proj, const int32_t* seq_lens,
                             const int32_t* page_table, int32_t max_pages_per_seq,
                             const int32_t* sel_pages, const int32_t* sel_phys,
                             const int32_t* sel_counts, int32_t k_max, float softmax_scale,
                             float* z_out, float* lse_out, void* workspace, size_t ws_bytes,
                             int32_t batch, void* stream);

/*
 * kvlr_decode_attn with the up-projection applied in its merge launch.
 * BasisKV English abstract and method details (key innovation): the value
 * latent is tied to the output projection, so o_h = z_h . B_v[g] is applied
 * once per query head, here by the workgroup that merges the head group's
 * chunk records (float32 FMA over rank_v terms).
 * Arguments as for kvlr_decode_attn, plus:
 *   factors  B_v is read ([H_kv][rank_v][head_dim], storage type)
 *   o_out    out [batch][num_q_heads][head_dim] float32 (required)
 * z_out and lse_out are written as by kvlr_decode_attn. o equals what
 * kvlr_upproject gives for the same z up to float32 summation order.
 */
kvlr_status kvlr_decode_attn_upproject(const kvlr_shape* shape, const kvlr_factors* factors,
                                       const kvlr_cache* cache, const float* q,
                                       const float* q_proj, const int32_t* seq_lens,
                                       const int32_t* page_table, int32_t max_pages_per_seq,
                                       const int32_t* sel_pages, const int32_t* sel_phys,
                                       const int32_t* sel_counts, int32_t k_max,
                                       float softmax_scale, float* z_out, float* lse_out,
                                       float* o_out, void* workspace, size_t ws_bytes,
                                       int32_t batch, void* stream);

/*
 * kvlr_decode_attn_upproject without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). Arguments, outputs and results
 * are those of kvlr_decode_attn_upproject (the same kernels), without
 * workspace and ws_bytes: the chunk records live in a static device array of
 * kvlr_noalloc_scratch_bytes() bytes (32 MiB) that each GPU the library runs
 * on holds until the process ends. A call needing more, i.e. batch * H_kv *
 * chunks * G * (rank_v + 2) * 4 bytes with chunks = ceil(rows / 16) for
 * selected pages (rows = k_max * page_size / 64) or ceil(rows / 128) for
 * every page (rows = max_pages_per_seq * page_size / 64), returns
 * KVLR_ERR_WORKSPACE_TOO_SMALL and enqueues nothing. The call allocates
 * nothing (no hipMalloc, no allocating library routine); its first use on a
 * device looks up that device's address of the array once. Every call on
 * one GPU shares the array: calls that overlap on one GPU (on different
 * streams, or from different threads) race and must be ordered by the
 * caller. Nothing in the array needs clearing: each chunk writes its record
 * before the merge launch reads it.
 */
kvlr_status kvlr_decode_attn_upproject_noalloc(const kvlr_shape* shape, const kvlr_factors* factors,
                                               const kvlr_cache* cache, const float* q,
                                               const float* q_proj, const int32_t* seq_lens,
                                               const int32_t* page_table, int32_t max_pages_per_seq,
                                               const int32_t* sel_pages, const int32_t* sel_phys,
                                               const int32_t* sel_counts, int32_t k_max,
                                               float softmax_scale, float* z_out, float* lse_out,
                                               float* o_out, int32_t batch, void* stream);

/* Bytes of the static scratch kvlr_decode_attn_upproject_noalloc uses. */
size_t kvlr_noalloc_scratch_bytes(void);

/*
 * Up-projection, once per query head. BasisKV English abstract and method
 * details: value compression is tied to the output projection, so the
 * decoder B_v is applied to the attention-weighted latent z.
 *   o_out[b][h] = z[b][h] . B_v[h / G]
 *   z      [batch][num_q_heads][rank_v] float32
 *   o_out  out [batch][num_q_heads][head_dim] float32
 * Float32 matrix cores, float32 accumulation.
 */
kvlr_status kvlr_upproject(const kvlr_shape* shape, const kvlr_factors* factors, const float* z,
                           float* o_out, int32_t batch, void* stream);

/*
 * Encode weight preparation. BasisKV English abstract (low-rank K/V
 * projections; the residual is what the value latent cannot predict of the
 * key): since (K - v W_pred) A_k = K A_k - v (W_pred A_k), the encode needs
 * W_pred and A_k only through their r_v x r_k product. kvlr_prepare_residual
 * forms -(W_pred A_k) once per factor set (float32 sums of exact products on
 * the matrix cores, then, for bf16, split into high and low bf16 parts) in
 * the operand layout the encode kernels read; pass it as
 * kvlr_factors.residual_prep. The encode's outputs are bit-identical with or
 * without it (the same arithmetic, done once instead of per workgroup).
 *   prep        out, device, 16-byte aligned, prep_bytes >= the size below
 * kvlr_residual_prep_bytes: its size for this shape (host); 0 when the shape
 * has no residual (KVLR_KEYS_LATENT) or is rejected.
 * Needs A_k and W_pred in factors; KVLR_KEYS_LATENT returns
 * KVLR_ERR_INVALID_ARGUMENT, a too small buffer KVLR_ERR_WORKSPACE_TOO_SMALL.
 */
size_t kvlr_residual_prep_bytes(const kvlr_shape* shape);
kvlr_status kvlr_prepare_residual(const kvlr_shape* shape, const kvlr_factors* factors,
                                  void* prep, size_t prep_bytes, void* stream);

/*
 * Page-table check, a debugging aid (not part of the decode step). The decode
 * calls trust the page tables: they read each sequence's length only up to
 * max_pages_per_seq * page_size tokens (never past its table row), but use the
 * entries as given. This call checks, on the device, each sequence b of the
 * batch: 0 <= seq_lens[b] <= max_pages_per_seq * page_size, and every entry
 * page_table[b][j] for j < ceil(min(seq_lens[b], max_pages_per_seq *
 * page_size) / page_size) within [0, shape->num_phys_pages).
 *   errors  out, device uint32 [2], 16-byte aligned, cleared by this call:
 *           errors[0] = KVLR_TABLE_ERR_* bits found, errors[1] = entries out
 *           of range. Asynchronous on `stream`: read them after it.
 */
#define KVLR_TABLE_ERR_PAGE 1u    /* an entry in use outside [0, num_phys_pages) */
#define KVLR_TABLE_ERR_LENGTH 2u  /* a length below 0 or above max_pages_per_seq * page_size */
kvlr_status kvlr_check_page_tables(const kvlr_shape* shape, const int32_t* seq_lens,
                                   const int32_t* page_table, int32_t max_pages_per_seq, int32_t batch,
                                   uint32_t* errors, void* stream);

/* Workspace bytes that route and attention need for this shape (host). */
size_t kvlr_workspace_bytes(const kvlr_shape* shape, int32_t batch, int32_t max_pages_per_seq);

/* Zero-fills a workspace with a kernel (no memset node), once after allocation. */
kvlr_status kvlr_workspace_init(void* workspace, size_t ws_bytes, void* stream);

/* Static text for a status; for KVLR_ERR_HIP, the text of the calling
 * thread's last HIP error (valid until that thread's next failing call). */
const char* kvlr_status_string(kvlr_status status);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int32_t kvlr_version(void);

/*
 * Output projection seen from the value latents. BasisKV English abstract and
 * method details (key innovation): value compression is tied to the output
 * projection, so the same low-rank value representation narrows both the
 * value cache and what the attention output carries. With o_h = z_h . B_v,
 *   W_o . concat_h(o_h) = F . concat_h(z_h),  F = W_o . blockdiag_h(B_v^T).
 * bf16 storage only (other types return KVLR_ERR_UNSUPPORTED).
 *
 * kvlr_fold_output_weights forms F once (a weight preparation):
 *   W_o    [hidden][num_q_heads * head_dim] bf16, rows are output features
 *   F_out  out [hidden][num_q_heads * rank_v] bf16 (RNE of float32 sums of
 *          exact bf16 products)
 *   hidden host; a positive multiple of 16, at most 2^20
 */
kvlr_status kvlr_fold_output_weights(const kvlr_shape* shape, const kvlr_factors* factors,
                                     const void* W_o, int32_t hidden, void* F_out, void* stream);

/*
 * kvlr_output_projection applies F to a batch of latent outputs:
 *   out[b] = F . z[b],  z [batch][num_q_heads][rank_v] float32 (read as one
 *   row of num_q_heads * rank_v), out [batch][hidden] float32.
 * z enters as bf16 high and low halves (about 16 significant bits), sums are
 * float32.
 */
kvlr_status kvlr_output_projection(const kvlr_shape* shape, const void* F, const float* z,
                                   int32_t hidden, float* out, int32_t batch, void* stream);

/*
 * Factor fitting from sample keys and values (calibration, not decode).
 * BasisKV English abstract (low-rank K/V projections; the value latent
 * predicts part of each key and a key-specific residual holds what the value
 * cannot recover) and method details (key design: the choice of the
 * low-rank factors). The pages leave the fit open; the library implements
 * the staged least-squares reading, per KV head g, from n samples
 * K, V [n][d]:
 *   A_v    = top-r_v eigenvectors of V^T V                 B_v = A_v^T
 *   W_pred = (v^T v)^-1 v^T K,  v = V . A_v                (exact keys only)
 *   A_k    = top-r_k eigenvectors of R^T R, R = K - v . W_pred  (exact keys)
 *            or of K^T K                                   (latent keys)
 *   B_k    = A_k^T
 * Eigenvectors come largest eigenvalue first, each scaled so that its entry
 * of largest magnitude is positive. All of it follows from the second
 * moments V^T V, K^T K and V^T K, which the GPU accumulates; the host solves
 * the d x d eigenproblems in float64.
 *
 * Samples k, v are [n][H_kv][head_dim] in the storage type (the layout of
 * kvlr_append_encode's new tokens); n is host, n <= 2^31 - 1. With exact
 * keys n should well exceed rank_v + rank_k: at n <= rank_v the value latent
 * reproduces the samples' keys exactly, the residual vanishes and A_k is
 * arbitrary.
 */
typedef struct kvlr_factor_buffers {
  void* A_v;     /* out [H_kv][head_dim][rank_v] */
  void* B_v;     /* out [H_kv][rank_v][head_dim] */
  void* A_k;     /* out [H_kv][head_dim][rank_k] */
  void* B_k;     /* out [H_kv][rank_k][head_dim] */
  void* W_pred;  /* out [H_kv][rank_v][head_dim], KVLR_KEYS_EXACT only */
} kvlr_factor_buffers;

/* Device workspace bytes for kvlr_fit_moments / kvlr_fit_factors with n
 * samples (at most about 100 MB plus the float64 moments); 0 for a rejected
 * shape. */
size_t kvlr_fit_workspace_bytes(const kvlr_shape* shape, int32_t n);

/*
 * Second moments of n samples, accumulated on the GPU (stream-ordered,
 * asynchronous like the decode calls):
 *   moments  device [H_kv][3][head_dim][head_dim] float64: V^T V, K^T K,
 *            V^T K per KV head. accumulate = 0 overwrites, 1 adds onto the
 *            buffer's contents, so calibration can stream batches of samples.
 * bf16 samples multiply exactly on the matrix cores with float32 sums over
 * runs of at least 2048 tokens (when n allows); f32 samples use float32
 * FMA. Runs are added in a fixed order in float64: results are
 * deterministic. n = 0 is a no-op (or zeroes the moments).
 */
kvlr_status kvlr_fit_moments(const kvlr_shape* shape, const void* k, const void* v, int32_t n,
                             double* moments, int32_t accumulate, void* workspace,
                             size_t ws_bytes, void* stream);

/*
 * Host only (touches no device): the factors from float64 moments.
 *   moments  host [H_kv][3][head_dim][head_dim] as kvlr_fit_moments writes
 *   A_v      host out [H_kv][head_dim][rank_v] float64 (B_v = A_v^T)
 *   A_k      host out [H_kv][head_dim][rank_k] float64 (B_k = A_k^T)
 *   W_pred   host out [H_kv][rank_v][head_dim] float64, KVLR_KEYS_EXACT only
 *   lam_v, lam_k  host out [H_kv][rank_v] / [H_kv][rank_k]: the eigenvalues
 *            of the chosen eigenvectors (may be NULL)
 * Returns KVLR_ERR_NUMERICAL when v^T v is numerically singular: a Cholesky
 * pivot at or below 1e-6 of its largest diagonal entry, i.e. a chosen value
 * direction with under a millionth of the leading direction's energy (below
 * the resolution of float32-accumulated moments). Uses up to 16 host threads
 * (one KV head each).
 */
kvlr_status kvlr_fit_solve(const kvlr_shape* shape, const double* moments, double* A_v,
                           double* A_k, double* W_pred, double* lam_v, double* lam_k);

/*
 * Host only: per-head residual ranks for an adaptive residual (see the
 * kvlr_cache.k_lat_ranks comment) from the fit's residual spectrum. For each
 * KV head g, ranks_out[g] is the smallest r in {16, 32, 64}, r <= rank_k,
 * whose top-r residual eigenvalues carry at least energy_frac of the energy
 * of the top rank_k (negative eigenvalues count as zero), else rank_k.
 *   lam_k     host [H_kv][rank_k], largest first (kvlr_fit_solve's lam_k)
 *   ranks_out host out [H_kv]
 * KVLR_KEYS_EXACT only; energy_frac in (0, 1].
 */
kvlr_status kvlr_choose_residual_ranks(const kvlr_shape* shape, const double* lam_k,
                                       double energy_frac, int32_t* ranks_out);

/*
 * The whole fit in one synchronous call: kvlr_fit_moments into the
 * workspace, a copy of the moments to the host, kvlr_fit_solve, and the
 * factors written to `out` in the storage type (RNE of the float32 value).
 * lam_v, lam_k as in kvlr_fit_solve (host, may be NULL). Unlike the decode
 * calls it synchronises `stream` and uses host memory (a few MB) and up to
 * 16 host threads; it is meant for calibration, not for the decode loop.
 */
kvlr_status kvlr_fit_factors(const kvlr_shape* shape, const void* k, const void* v, int32_t n,
                             const kvlr_factor_buffers* out, double* lam_v, double* lam_k,
                             void* workspace, size_t ws_bytes, void* stream);

/*
 * Joint fit of the value decoders across attention partitions (calibration,
 * not decode). BasisKV English abstract: the low-rank factors are optimised
 * jointly across the per-GPU attention partitions against the complete
 * attention output, rather than fitting each partition on its own; method
 * details (key design: the loss couples every GPU's attention partition;
 * key innovation: value compression is tied to the output projection).
 * The pages give no procedure; the reading implemented here keeps the value
 * encoders A_v as fitted (the cache's latents exist before any query) and
 * chooses the decoder of the complete attention output from the latents of
 * every partition by least squares over calibration samples:
 *   z_h = x_h . A_v[h / G]           latent output of query head h
 *   D   = argmin sum_n |x_n - z_n D|^2 = (Z^T Z)^-1 Z^T X
 *   F   = W_o . D^T                   the output projection seen from the
 *                                     latents (as kvlr_fold_output_weights,
 *                                     whose F is this with D = blockdiag(B_v))
 * x_n = concat_h(x_h) [H_q * head_dim] is one sample's exact attention output
 * (all query heads of all partitions), z_n [H_q * rank_v] its latents. For
 * any W_o, F minimises sum_n |W_o x_n - F z_n|^2. Sizes: H_q * rank_v <=
 * 4096 and H_q * head_dim <= 16384; bf16 or f32 storage (not FP8 latents);
 * n should well exceed H_q * rank_v.
 *   x        [n][num_q_heads][head_dim] float32 samples (device)
 *   factors  A_v is read ([H_kv][head_dim][rank_v], storage type)
 */
size_t kvlr_fit_joint_workspace_bytes(const kvlr_shape* shape, int32_t n);

/* The moments of n samples, accumulated on the GPU (stream-ordered):
 *   zz  device [H_q rank_v][H_q rank_v] float64: Z^T Z
 *   zx  device [H_q rank_v][H_q head_dim] float64: Z^T X
 * accumulate = 1 adds onto zz, zx (streamed calibration), 0 overwrites.
 * Z is formed in float32 on the matrix cores; the moments take float32 sums
 * over runs of 256 samples and float64 sums of the runs. */
kvlr_status kvlr_fit_joint_moments(const kvlr_shape* shape, const kvlr_factors* factors,
                                   const float* x, int32_t n, double* zz, double* zx,
                                   int32_t accumulate, void* workspace, size_t ws_bytes,
                                   void* stream);

/* Host only: D = zz^-1 zx in float64 (Cholesky, then the triangular solves
 * for each of the H_q head_dim columns on up to 16 host threads).
 *   zz, zx  host, as kvlr_fit_joint_moments writes them
 *   D_out   host out [H_q rank_v][H_q head_dim] float64
 * KVLR_ERR_NUMERICAL when a Cholesky pivot falls to 1e-12 of the largest
 * diagonal entry (latents the samples do not determine). */
kvlr_status kvlr_fit_joint_solve(const kvlr_shape* shape, const double* zz, const double* zx,
                                 double* D_out);

/* F = W_o . D^T on the GPU (bf16 storage only):
 *   W_o    [hidden][H_q head_dim] bf16, rows are output features
 *   D      [H_q rank_v][H_q head_dim] float32 (device)
 *   F_out  out [hidden][H_q rank_v] bf16 (RNE of float32 sums of float32
 *          products, summed in float64 over runs of 256)
 * F_out is what kvlr_output_projection applies. */
kvlr_status kvlr_fold_joint_decoder(const kvlr_shape* shape, const void* W_o, int32_t hidden,
                                    const float* D, void* F_out, void* stream);

/* The whole joint fit in one synchronous call: the moments into the
 * workspace, a copy to the host, the solve, D rounded to float32 and folded
 * into F_out. D_out (host, may be NULL) receives the float64 decoder. Uses
 * host memory (about 3 (H_q rank_v)^2 + 3 H_q rank_v H_q head_dim doubles)
 * and synchronises `stream`: for calibration, not the decode loop. */
kvlr_status kvlr_fit_joint(const kvlr_shape* shape, const kvlr_factors* factors, const float* x,
                           int32_t n, const void* W_o, int32_t hidden, void* F_out, double* D_out,
                           void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVLR_H */
