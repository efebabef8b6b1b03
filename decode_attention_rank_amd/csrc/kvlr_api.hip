// C-ABI entry points: host-side validation, workspace layout, dispatch.
// Nothing here touches the GPU before every argument has been checked, so a
// rejected call enqueues nothing.

#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "kvlr.h"
#include "kvlr_internal.h"

// Chunk-record scratch of kvlr_decode_attn_upproject_noalloc: one copy per
// GPU, held until the process ends. Host code never passes this name to a
// kernel (on the host it only stands for the symbol); it uses the device
// address that hipGetSymbolAddress returns for the current device.
static constexpr size_t kStaticScratchBytes = static_cast<size_t>(32) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch`, per device

using kvlr::Dims;

thread_local char g_hip_msg[256] = "no HIP error recorded";

kvlr_status hip_status(hipError_t e) {
  if (e == hipSuccess) return KVLR_OK;
  snprintf(g_hip_msg, sizeof(g_hip_msg), "HIP error %d: %s", static_cast<int>(e), hipGetErrorString(e));
  return KVLR_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
bool one_of(int v, int a, int b, int c) { return v == a || v == b || v == c; }

// Checks the shape; fills Dims on success.
kvlr_status check_shape(const kvlr_shape* s, Dims* dm) {
  if (!s) return KVLR_ERR_INVALID_ARGUMENT;
  if (s->num_q_heads < 1 || s->num_kv_heads < 1 || s->head_dim < 1 || s->page_size < 1 ||
      s->rank_v < 1 || s->rank_k < 1 || s->num_phys_pages < 1)
    return KVLR_ERR_INVALID_ARGUMENT;
  if (s->num_q_heads % s->num_kv_heads != 0) return KVLR_ERR_INVALID_ARGUMENT;
  if (s->dtype != KVLR_DTYPE_BF16 && s->dtype != KVLR_DTYPE_F32 && s->dtype != KVLR_DTYPE_BF16_FP8)
    return KVLR_ERR_INVALID_ARGUMENT;
  if (s->key_mode != KVLR_KEYS_LATENT && s->key_mode != KVLR_KEYS_EXACT) return KVLR_ERR_INVALID_ARGUMENT;
  if (s->rank_v > s->head_dim || s->rank_k > s->head_dim) return KVLR_ERR_INVALID_ARGUMENT;
  const int G = s->num_q_heads / s->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVLR_ERR_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return KVLR_ERR_UNSUPPORTED;
  // rank_v may be the full head_dim 128 (values stored uncompressed); rank_k <= 64
  if (!(one_of(s->rank_v, 16, 32, 64) || s->rank_v == 128) || !one_of(s->rank_k, 16, 32, 64))
    return KVLR_ERR_UNSUPPORTED;
  if (s->rank_v == 128 && s->dtype != KVLR_DTYPE_BF16) return KVLR_ERR_UNSUPPORTED;
  if (!one_of(s->page_size, 16, 32, 64)) return KVLR_ERR_UNSUPPORTED;
  // FP8 latents run on the matrix-core paths, which take one 64-token page per row
  if (s->dtype == KVLR_DTYPE_BF16_FP8 && s->page_size != 64) return KVLR_ERR_UNSUPPORTED;
  dm->Hq = s->num_q_heads;
  dm->Hkv = s->num_kv_heads;
  dm->G = G;
  dm->D = s->head_dim;
  dm->P = s->page_size;
  dm->RV = s->rank_v;
  dm->RK = s->rank_k;
  dm->dtype = s->dtype == KVLR_DTYPE_F32 ? 1 : 0;   // factors, original keys, new tokens
  dm->lat = s->dtype == KVLR_DTYPE_BF16_FP8 ? 2 : dm->dtype;
  dm->exact = s->key_mode == KVLR_KEYS_EXACT ? 1 : 0;
  return KVLR_OK;
}

// The current device's address of the static scratch, looked up once per
// device (with that device current) and kept.
kvlr_status static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return KVLR_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return KVLR_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return KVLR_OK;
}

constexpr size_t kAlign = 256;
constexpr int kMaxBatch = 4096;          // per-sequence offsets and work lists live in LDS
#ifndef KVLR_ROUTE_GRID
#define KVLR_ROUTE_GRID 2048
#endif
constexpr long long kPersistentGrid = KVLR_ROUTE_GRID;  // about 8 workgroups per CU
#ifndef KVLR_ROUTE_STATIC
#define KVLR_ROUTE_STATIC 1  // fixed chunks per pair when one workgroup per chunk fits the grid
#endif
#ifndef KVLR_ATTN_GRID
#define KVLR_ATTN_GRID 1024
#endif
constexpr long long kAttnGrid = KVLR_ATTN_GRID;        // attention holds more registers per wave
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int ceil_div(long long a, long long b) { return static_cast<int>((a + b - 1) / b); }

// Workspace plan. Route: [tickets | scores]; attention: [chunk partials].
struct Plan {
  size_t route_cnt, route_scores, attn_part, total;
  int attn_max_splits;
};

int attn_rows(int n_items, int P) { return ceil_div(n_items, 64 / P); }
int max_chunks(int rows, int rows_per_chunk) {
  const int c = ceil_div(rows, rows_per_chunk);
  return c > 1 ? c : 1;
}

Plan plan_for(const Dims& dm, int batch, int max_pages) {
  Plan p{};
  const size_t pairs = static_cast<size_t>(batch) * dm.Hkv;
  size_t off = 0;
  if (dm.exact) {
    p.route_cnt = off;
    off += round_up(pairs * sizeof(uint32_t));
    p.route_scores = off;
    off += round_up(pairs * static_cast<size_t>(max_pages) * sizeof(float));
  }
  // partial slots per pair: enough for the smallest chunk size over every page
  p.attn_max_splits = max_chunks(attn_rows(max_pages, dm.P), kvlr::attn_rows_per_chunk(true));
  p.attn_part = off;
  off += round_up(pairs * p.attn_max_splits * dm.G * static_cast<size_t>(dm.RV + 2) * sizeof(float));
  p.total = off;
  return p;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Bytes of one 64-token routing row holding `width` latent elements per token.
int route_row_bytes(const Dims& dm, int width) {
  const int elem = dm.lat == 2 ? 1 : dm.lat == 1 ? 4 : 2;
  return 64 * width * elem;
}

// Residual-latent layout from the cache's per-head rank table (NULL:
// uniform). Per-head ranks need routed keys, 64-token pages, bf16 keys and
// bf16 or FP8 latents, at most kMaxAdaptiveHeads KV heads, and each rank in
// {16, 32, 64} and at most rank_k.
kvlr_status residual_layout(const Dims& dm, const kvlr_cache* cache, kvlr::KLayout* kl) {
  *kl = kvlr::KLayout{};
  if (!cache->k_lat_ranks) return KVLR_OK;
  if (!dm.exact || dm.P != 64 || dm.dtype != 0 || dm.Hkv > kvlr::kMaxAdaptiveHeads)
    return KVLR_ERR_UNSUPPORTED;
  kl->adaptive = 1;
  int off = 0;
  for (int g = 0; g < dm.Hkv; ++g) {
    const int r = cache->k_lat_ranks[g];
    if (!one_of(r, 16, 32, 64) || r > dm.RK) return KVLR_ERR_INVALID_ARGUMENT;
    kl->ck[g] = r / 8;  // 8 elements per chunk for bf16 and FP8 latents
    kl->off[g] = off;
    off += kl->ck[g];
  }
  kl->page_chunks = off;
  // routing work chunks of equal bytes: rows per chunk scaled by the
  // smallest head's (rank_v + r) over this head's
  int rmin = 64;
  for (int g = 0; g < dm.Hkv; ++g) rmin = cache->k_lat_ranks[g] < rmin ? cache->k_lat_ranks[g] : rmin;
  for (int g = 0; g < dm.Hkv; ++g) {
    const int rpc = kvlr::route_rows_per_chunk(route_row_bytes(dm, dm.RV + rmin)) * (dm.RV + rmin) /
                    (dm.RV + cache->k_lat_ranks[g]);
    kl->rpc[g] = rpc > 1 ? rpc : 1;
  }
  return KVLR_OK;
}

}  // namespace

extern "C" {

int32_t kvlr_version(void) { return 100; }

const char* kvlr_status_string(kvlr_status st) {
  switch (st) {
    case KVLR_OK: return "ok";
    case KVLR_ERR_INVALID_ARGUMENT: return "invalid argument";
    case KVLR_ERR_UNSUPPORTED: return "unsupported shape";
    case KVLR_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KVLR_ERR_HIP: return g_hip_msg;
    case KVLR_ERR_NUMERICAL: return "the fit's linear algebra failed (rank-deficient samples)";
  }
  return "unknown status";
}

int32_t kvlr_qproj_width(const kvlr_shape* shape) {
  Dims dm;
  if (check_shape(shape, &dm) != KVLR_OK) return 0;
  return dm.exact ? dm.RV + dm.RK : dm.RK;
}

size_t kvlr_workspace_bytes(const kvlr_shape* shape, int32_t batch, int32_t max_pages_per_seq) {
  Dims dm;
  if (check_shape(shape, &dm) != KVLR_OK || batch < 0 || max_pages_per_seq < 1 ||
      max_pages_per_seq > 65536)
    return 0;
  return plan_for(dm, batch, max_pages_per_seq).total;
}

kvlr_status kvlr_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
  if (ws_bytes == 0) return KVLR_OK;
  if (!ok_ptr(workspace)) return KVLR_ERR_INVALID_ARGUMENT;
  return hip_status(kvlr::launch_zero_fill(workspace, ws_bytes, as_stream(stream)));
}

// Checks the append's buffers and fills the encode part of *a (total_new > 0).
static kvlr_status encode_args(const Dims& dm, const kvlr_factors* factors, const kvlr_cache* cache,
                               const void* k_new, const void* v_new, const int32_t* cu_new,
                               const int32_t* seq_lens_before, const int32_t* page_table,
                               int32_t max_pages_per_seq, int32_t batch, int32_t total_new,
                               kvlr::EncodeArgs* a) {
  if (!ok_ptr(factors->A_v) || !ok_ptr(factors->A_k) || !ok_ptr(cache->v_lat) ||
      !ok_ptr(cache->k_lat) || !ok_ptr(k_new) || !ok_ptr(v_new) || !ok_ptr(cu_new) ||
      !ok_ptr(seq_lens_before) || !ok_ptr(page_table))
    return KVLR_ERR_INVALID_ARGUMENT;
  if (dm.exact && (!ok_ptr(factors->W_pred) || !ok_ptr(cache->k_exact))) return KVLR_ERR_INVALID_ARGUMENT;
  if (dm.exact && factors->residual_prep && !aligned16(factors->residual_prep))
    return KVLR_ERR_INVALID_ARGUMENT;
  const kvlr_status st = residual_layout(dm, cache, &a->kl);
  if (st != KVLR_OK) return st;
  a->dm = dm;
  a->A_v = factors->A_v;
  a->A_k = factors->A_k;
  a->W_pred = factors->W_pred;
  a->m_prep = dm.exact ? factors->residual_prep : nullptr;
  a->k_new = k_new;
  a->v_new = v_new;
  a->cu_new = cu_new;
  a->lens_before = seq_lens_before;
  a->page_table = page_table;
  a->max_pages = max_pages_per_seq;
  a->v_lat = cache->v_lat;
  a->k_lat = cache->k_lat;
  a->k_exact = cache->k_exact;
  a->batch = batch;
  a->total_new = total_new;
  return KVLR_OK;
}

kvlr_status kvlr_append_encode(const kvlr_shape* shape, const kvlr_factors* factors,
                               const kvlr_cache* cache, const void* k_new, const void* v_new,
                               const int32_t* cu_new, const int32_t* seq_lens_before,
                               const int32_t* page_table, int32_t max_pages_per_seq,
                               int32_t batch, int32_t total_new, void* stream) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  if (!factors || !cache || batch < 0 || total_new < 0) return KVLR_ERR_INVALID_ARGUMENT;
  if (max_pages_per_seq < 1 || max_pages_per_seq > 65536) return KVLR_ERR_INVALID_ARGUMENT;
  if (batch == 0 || total_new == 0) return KVLR_OK;
  if (batch > kMaxBatch) return KVLR_ERR_UNSUPPORTED;
  kvlr::EncodeArgs a{};
  st = encode_args(dm, factors, cache, k_new, v_new, cu_new, seq_lens_before, page_table,
                   max_pages_per_seq, batch, total_new, &a);
  if (st != KVLR_OK) return st;
  return hip_status(kvlr::launch_encode(a, as_stream(stream)));
}

kvlr_status kvlr_append_encode_project(const kvlr_shape* shape, const kvlr_factors* factors,
                                       const kvlr_cache* cache, const void* k_new,
                                       const void* v_new, const int32_t* cu_new,
                                       const int32_t* seq_lens_before, const int32_t* page_table,
                                       int32_t max_pages_per_seq, int32_t batch, int32_t total_new,
                                       const float* q, float* q_proj, void* stream) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  if (!factors || !cache || batch < 0 || total_new < 0) return KVLR_ERR_INVALID_ARGUMENT;
  if (max_pages_per_seq < 1 || max_pages_per_seq > 65536) return KVLR_ERR_INVALID_ARGUMENT;
  if (batch == 0) return KVLR_OK;
  if (batch > kMaxBatch) return KVLR_ERR_UNSUPPORTED;
  if (!ok_ptr(factors->B_k) || !ok_ptr(q) || !ok_ptr(q_proj)) return KVLR_ERR_INVALID_ARGUMENT;
  if (dm.exact && !ok_ptr(factors->W_pred)) return KVLR_ERR_INVALID_ARGUMENT;
  kvlr::EncodeArgs a{};
  if (total_new > 0) {
    st = encode_args(dm, factors, cache, k_new, v_new, cu_new, seq_lens_before, page_table,
                     max_pages_per_seq, batch, total_new, &a);
    if (st != KVLR_OK) return st;
  } else {
    a.dm = dm;
    a.W_pred = factors->W_pred;
    a.batch = batch;
  }
  a.B_k = factors->B_k;
  a.q = q;
  a.q_proj = q_proj;
  return hip_status(kvlr::launch_encode(a, as_stream(stream)));
}

size_t kvlr_residual_prep_bytes(const kvlr_shape* shape) {
  Dims dm;
  if (check_shape(shape, &dm) != KVLR_OK || !dm.exact) return 0;
  return kvlr::encode_prep_bytes(dm);
}

kvlr_status kvlr_prepare_residual(const kvlr_shape* shape, const kvlr_factors* factors, void* prep,
                                  size_t prep_bytes, void* stream) {
  Dims dm;
  const kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  if (!factors || !dm.exact || !ok_ptr(factors->A_k) || !ok_ptr(factors->W_pred) || !ok_ptr(prep))
    return KVLR_ERR_INVALID_ARGUMENT;
  const size_t need = kvlr::encode_prep_bytes(dm);
  if (need == 0) return KVLR_ERR_UNSUPPORTED;
  if (prep_bytes < need) return KVLR_ERR_WORKSPACE_TOO_SMALL;
  kvlr::EncodeArgs a{};
  a.dm = dm;
  a.A_v = factors->A_v;
  a.A_k = factors->A_k;
  a.W_pred = factors->W_pred;
  return hip_status(kvlr::launch_encode_prep(a, prep, as_stream(stream)));
}

kvlr_status kvlr_check_page_tables(const kvlr_shape* shape, const int32_t* seq_lens,
                                   const int32_t* page_table, int32_t max_pages_per_seq, int32_t batch,
                                   uint32_t* errors, void* stream) {
  Dims dm;
  const kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  if (batch < 0 || batch > kMaxBatch || max_pages_per_seq < 1 || max_pages_per_seq > 65536 ||
      !ok_ptr(errors) || (batch > 0 && (!ok_ptr(seq_lens) || !ok_ptr(page_table))))
    return KVLR_ERR_INVALID_ARGUMENT;
  return hip_status(kvlr::launch_check_tables(seq_lens, page_table, max_pages_per_seq, dm.P,
                                              shape->num_phys_pages, batch, errors, as_stream(stream)));
}

kvlr_status kvlr_project_queries(const kvlr_shape* shape, const kvlr_factors* factors,
                                 const float* q, float* q_proj, int32_t batch, void* stream) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  if (!factors || batch < 0) return KVLR_ERR_INVALID_ARGUMENT;
  if (batch == 0) return KVLR_OK;
  if (!ok_ptr(factors->B_k) || !ok_ptr(q) || !ok_ptr(q_proj)) return KVLR_ERR_INVALID_ARGUMENT;
  if (dm.exact && !ok_ptr(factors->W_pred)) return KVLR_ERR_INVALID_ARGUMENT;
  kvlr::QprojArgs a{};
  a.dm = dm;
  a.W_pred = factors->W_pred;
  a.B_k = factors->B_k;
  a.q = q;
  a.q_proj = q_proj;
  a.batch = batch;
  return hip_status(kvlr::launch_qproj(a, as_stream(stream)));
}

// Routing: page scores, and unless scores_only the fused top-k selection.
static kvlr_status route_impl(const kvlr_shape* shape, const kvlr_cache* cache, const float* q_proj,
                              const int32_t* seq_lens, const int32_t* page_table,
                              int32_t max_pages_per_seq, int32_t topk_num, int32_t topk_den,
                              const int32_t* k_pages, int32_t k_max, int32_t* sel_pages,
                              int32_t* sel_counts, int32_t* sel_phys, float* page_scores,
                              void* workspace, size_t ws_bytes, int32_t batch, void* stream,
                              bool scores_only) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  if (!dm.exact) return KVLR_ERR_UNSUPPORTED;
  if (dm.RV > 64) return KVLR_ERR_UNSUPPORTED;  // routing reads compressed value latents
  if (!cache || batch < 0) return KVLR_ERR_INVALID_ARGUMENT;
  if (batch > kMaxBatch) return KVLR_ERR_UNSUPPORTED;
  if (max_pages_per_seq < 1 || max_pages_per_seq > 65536) return KVLR_ERR_INVALID_ARGUMENT;
  if (scores_only) {
    // no selection: only the scores are written
  } else if (k_pages) {
    // per-sequence budgets: the caller keeps each within [0, k_max]
    if (k_max < 1 || k_max > max_pages_per_seq || !aligned16(k_pages)) return KVLR_ERR_INVALID_ARGUMENT;
  } else {
    if (topk_num < 0 || topk_den < 1) return KVLR_ERR_INVALID_ARGUMENT;
    const long long bound = (static_cast<long long>(max_pages_per_seq) * topk_num + topk_den - 1) / topk_den;
    const long long need_k = bound < 1 ? 1 : (bound > max_pages_per_seq ? max_pages_per_seq : bound);
    if (k_max < need_k || k_max > max_pages_per_seq) return KVLR_ERR_INVALID_ARGUMENT;
  }
  if (batch == 0) return KVLR_OK;
  if (!ok_ptr(cache->v_lat) || !ok_ptr(cache->k_lat) || !ok_ptr(q_proj) || !ok_ptr(seq_lens) ||
      !ok_ptr(page_table))
    return KVLR_ERR_INVALID_ARGUMENT;
  if (scores_only ? !ok_ptr(page_scores) : (!ok_ptr(sel_pages) || !ok_ptr(workspace)))
    return KVLR_ERR_INVALID_ARGUMENT;
  if (page_scores && !aligned16(page_scores)) return KVLR_ERR_INVALID_ARGUMENT;
  if (sel_counts && !aligned16(sel_counts)) return KVLR_ERR_INVALID_ARGUMENT;
  if (sel_phys && !aligned16(sel_phys)) return KVLR_ERR_INVALID_ARGUMENT;
  const Plan plan = plan_for(dm, batch, max_pages_per_seq);
  if (!scores_only && ws_bytes < plan.total) return KVLR_ERR_WORKSPACE_TOO_SMALL;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  kvlr::RouteArgs a{};
  a.scores_only = scores_only ? 1 : 0;
  st = residual_layout(dm, cache, &a.kl);
  if (st != KVLR_OK) return st;
  a.dm = dm;
  a.v_lat = cache->v_lat;
  a.k_lat = cache->k_lat;
  a.q_proj = q_proj;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.max_pages = max_pages_per_seq;
  a.topk_num = topk_num;
  a.topk_den = topk_den;
  a.k_pages = k_pages;
  a.k_max = k_max;
  a.sel = sel_pages;
  a.sel_counts = sel_counts;
  a.sel_phys = sel_phys;
  a.scores = page_scores ? page_scores : reinterpret_cast<float*>(ws + plan.route_scores);
  a.counters = scores_only ? nullptr : reinterpret_cast<uint32_t*>(ws + plan.route_cnt);
  a.batch = batch;
  const int max_rows = ceil_div(static_cast<long long>(max_pages_per_seq) * dm.P, 64);
  a.rows_per_chunk = kvlr::route_rows_per_chunk(route_row_bytes(dm, dm.RV + dm.RK));
  long long chunks = 0;
  for (int g = 0; g < dm.Hkv; ++g) {
    const int rpc = a.kl.adaptive ? a.kl.rpc[g] : a.rows_per_chunk;
    chunks += static_cast<long long>(batch) * (max_rows > 0 ? ceil_div(max_rows, rpc) : 1);
  }
  a.grid = static_cast<int>(chunks < kPersistentGrid ? chunks : kPersistentGrid);
  // every pair sized for the widest table row when that fits one workgroup
  // per chunk: chunks of shorter sequences then only take their ticket
  // (with per-head ranks the kernel splits the table's rows per head)
  a.static_splits = (KVLR_ROUTE_STATIC && chunks <= kPersistentGrid && max_rows > 0)
                        ? (a.kl.adaptive ? max_rows : ceil_div(max_rows, a.rows_per_chunk)) : 0;
  return hip_status(kvlr::launch_route(a, as_stream(stream)));
}

kvlr_status kvlr_route_pages(const kvlr_shape* shape, const kvlr_cache* cache, const float* q_proj,
                             const int32_t* seq_lens, const int32_t* page_table,
                             int32_t max_pages_per_seq, int32_t topk_num, int32_t topk_den,
                             const int32_t* k_pages, int32_t k_max, int32_t* sel_pages,
                             int32_t* sel_counts, int32_t* sel_phys, float* page_scores,
                             void* workspace, size_t ws_bytes, int32_t batch, void* stream) {
  return route_impl(shape, cache, q_proj, seq_lens, page_table, max_pages_per_seq, topk_num,
                    topk_den, k_pages, k_max, sel_pages, sel_counts, sel_phys, page_scores,
                    workspace, ws_bytes, batch, stream, false);
}

kvlr_status kvlr_select_pages(const kvlr_shape* shape, const int32_t* seq_lens,
                              const int32_t* page_table, int32_t max_pages_per_seq,
                              float* page_scores, int32_t topk_num, int32_t topk_den,
                              const int32_t* k_pages, int32_t k_max, int32_t* sel_pages,
                              int32_t* sel_counts, int32_t* sel_phys, int32_t batch, void* stream) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  if (batch < 0) return KVLR_ERR_INVALID_ARGUMENT;
  if (batch > kMaxBatch) return KVLR_ERR_UNSUPPORTED;
  if (max_pages_per_seq < 1 || max_pages_per_seq > 65536) return KVLR_ERR_INVALID_ARGUMENT;
  if (k_pages) {
    if (k_max < 1 || k_max > max_pages_per_seq || !aligned16(k_pages)) return KVLR_ERR_INVALID_ARGUMENT;
  } else {
    if (topk_num < 0 || topk_den < 1) return KVLR_ERR_INVALID_ARGUMENT;
    const long long bound = (static_cast<long long>(max_pages_per_seq) * topk_num + topk_den - 1) / topk_den;
    const long long need_k = bound < 1 ? 1 : (bound > max_pages_per_seq ? max_pages_per_seq : bound);
    if (k_max < need_k || k_max > max_pages_per_seq) return KVLR_ERR_INVALID_ARGUMENT;
  }
  if (batch == 0) return KVLR_OK;
  if (!ok_ptr(seq_lens) || !ok_ptr(page_table) || !ok_ptr(page_scores) || !ok_ptr(sel_pages))
    return KVLR_ERR_INVALID_ARGUMENT;
  if (sel_counts && !aligned16(sel_counts)) return KVLR_ERR_INVALID_ARGUMENT;
  if (sel_phys && !aligned16(sel_phys)) return KVLR_ERR_INVALID_ARGUMENT;
  kvlr::RouteArgs a{};
  a.dm = dm;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.max_pages = max_pages_per_seq;
  a.topk_num = topk_num;
  a.topk_den = topk_den;
  a.k_pages = k_pages;
  a.k_max = k_max;
  a.sel = sel_pages;
  a.sel_counts = sel_counts;
  a.sel_phys = sel_phys;
  a.scores = page_scores;
  a.batch = batch;
  return hip_status(kvlr::launch_select(a, as_stream(stream)));
}

kvlr_status kvlr_score_pages(const kvlr_shape* shape, const kvlr_cache* cache, const float* q_proj,
                             const int32_t* seq_lens, const int32_t* page_table,
                             int32_t max_pages_per_seq, float* page_scores, int32_t batch,
                             void* stream) {
  return route_impl(shape, cache, q_proj, seq_lens, page_table, max_pages_per_seq, 1, 1, nullptr,
                    1, nullptr, nullptr, nullptr, page_scores, nullptr, 0, batch, stream, true);
}

static kvlr_status decode_attn_impl(const kvlr_shape* shape, const kvlr_factors* factors,
                                    const kvlr_cache* cache, const float* q, const float* q_proj,
                                    const int32_t* seq_lens, const int32_t* page_table,
                                    int32_t max_pages_per_seq, const int32_t* sel_pages,
                                    const int32_t* sel_phys, const int32_t* sel_counts,
                                    int32_t k_max, float softmax_scale, float* z_out,
                                    float* lse_out, float* o_out, void* workspace,
                                    size_t ws_bytes, int32_t batch, void* stream,
                                    bool use_static = false) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  if (!cache || batch < 0) return KVLR_ERR_INVALID_ARGUMENT;
  if (batch > kMaxBatch) return KVLR_ERR_UNSUPPORTED;
  if (max_pages_per_seq < 1 || max_pages_per_seq > 65536) return KVLR_ERR_INVALID_ARGUMENT;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return KVLR_ERR_INVALID_ARGUMENT;
  if (sel_pages && (k_max < 1 || k_max > max_pages_per_seq)) return KVLR_ERR_INVALID_ARGUMENT;
  if (batch == 0) return KVLR_OK;
  if (!ok_ptr(cache->v_lat) || !ok_ptr(seq_lens) || !ok_ptr(page_table) || !ok_ptr(z_out) ||
      (!use_static && !ok_ptr(workspace)))
    return KVLR_ERR_INVALID_ARGUMENT;
  if (sel_pages && !aligned16(sel_pages)) return KVLR_ERR_INVALID_ARGUMENT;
  if (sel_counts && (!sel_pages || !aligned16(sel_counts))) return KVLR_ERR_INVALID_ARGUMENT;
  if (sel_phys && (!sel_pages || !aligned16(sel_phys))) return KVLR_ERR_INVALID_ARGUMENT;
  if (lse_out && !aligned16(lse_out)) return KVLR_ERR_INVALID_ARGUMENT;
  if (dm.exact && (!ok_ptr(cache->k_exact) || !ok_ptr(q))) return KVLR_ERR_INVALID_ARGUMENT;
  if (o_out && (!factors || !ok_ptr(factors->B_v) || !aligned16(o_out))) return KVLR_ERR_INVALID_ARGUMENT;
  if (!dm.exact && (!ok_ptr(cache->k_lat) || !ok_ptr(q_proj))) return KVLR_ERR_INVALID_ARGUMENT;
  const Plan plan = plan_for(dm, batch, max_pages_per_seq);
  if (!use_static && ws_bytes < plan.total) return KVLR_ERR_WORKSPACE_TOO_SMALL;
  kvlr::AttnArgs a{};
  a.dm = dm;
  a.keys = dm.exact ? cache->k_exact : cache->k_lat;
  a.v_lat = cache->v_lat;
  a.qsrc = dm.exact ? q : q_proj;
  a.q_stride = dm.exact ? dm.D : dm.RK;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.max_pages = max_pages_per_seq;
  a.sel = sel_pages;
  a.sel_phys = sel_phys;
  a.sel_counts = sel_counts;
  a.k_max = sel_pages ? k_max : 0;
  a.scale_log2e = softmax_scale * 1.4426950408889634f;
  a.z_out = z_out;
  a.lse_out = lse_out;
  a.B_v = o_out ? factors->B_v : nullptr;
  a.o_out = o_out;
  a.batch = batch;
  const int rows = attn_rows(sel_pages ? k_max : max_pages_per_seq, dm.P);
  a.rows_per_chunk = kvlr::attn_rows_per_chunk(sel_pages != nullptr);
  a.max_splits = max_chunks(rows, a.rows_per_chunk);
  if (a.max_splits > plan.attn_max_splits) return KVLR_ERR_WORKSPACE_TOO_SMALL;
  if (use_static) {
    // this call's chunk records: pairs x chunks x (m, l, z) per query head
    const size_t need = static_cast<size_t>(batch) * dm.Hkv * a.max_splits * dm.G *
                        static_cast<size_t>(dm.RV + 2) * sizeof(float);
    if (need > kStaticScratchBytes) return KVLR_ERR_WORKSPACE_TOO_SMALL;
    void* p = nullptr;
    const kvlr_status sst = static_scratch(&p);
    if (sst != KVLR_OK) return sst;
    a.partials = static_cast<float*>(p);
  } else {
    a.partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + plan.attn_part);
  }
  const long long chunks = static_cast<long long>(batch) * dm.Hkv * a.max_splits;
  a.grid = static_cast<int>(chunks < kAttnGrid ? chunks : kAttnGrid);
  return hip_status(kvlr::launch_attn(a, as_stream(stream)));
}

kvlr_status kvlr_decode_attn(const kvlr_shape* shape, const kvlr_cache* cache, const float* q,
                             const float* q_proj, const int32_t* seq_lens,
                             const int32_t* page_table, int32_t max_pages_per_seq,
                             const int32_t* sel_pages, const int32_t* sel_phys,
                             const int32_t* sel_counts, int32_t k_max, float softmax_scale,
                             float* z_out, float* lse_out, void* workspace, size_t ws_bytes,
                             int32_t batch, void* stream) {
  return decode_attn_impl(shape, nullptr, cache, q, q_proj, seq_lens, page_table, max_pages_per_seq,
                          sel_pages, sel_phys, sel_counts, k_max, softmax_scale, z_out, lse_out,
                          nullptr, workspace, ws_bytes, batch, stream);
}

kvlr_status kvlr_decode_attn_upproject(const kvlr_shape* shape, const kvlr_factors* factors,
                                       const kvlr_cache* cache, const float* q,
                                       const float* q_proj, const int32_t* seq_lens,
                                       const int32_t* page_table, int32_t max_pages_per_seq,
                                       const int32_t* sel_pages, const int32_t* sel_phys,
                                       const int32_t* sel_counts, int32_t k_max,
                                       float softmax_scale, float* z_out, float* lse_out,
                                       float* o_out, void* workspace, size_t ws_bytes,
                                       int32_t batch, void* stream) {
  if (!o_out) return KVLR_ERR_INVALID_ARGUMENT;
  return decode_attn_impl(shape, factors, cache, q, q_proj, seq_lens, page_table,
                          max_pages_per_seq, sel_pages, sel_phys, sel_counts, k_max, softmax_scale,
                          z_out, lse_out, o_out, workspace, ws_bytes, batch, stream);
}

kvlr_status kvlr_decode_attn_upproject_noalloc(const kvlr_shape* shape, const kvlr_factors* factors,
                                               const kvlr_cache* cache, const float* q,
                                               const float* q_proj, const int32_t* seq_lens,
                                               const int32_t* page_table, int32_t max_pages_per_seq,
                                               const int32_t* sel_pages, const int32_t* sel_phys,
                                               const int32_t* sel_counts, int32_t k_max,
                                               float softmax_scale, float* z_out, float* lse_out,
                                               float* o_out, int32_t batch, void* stream) {
  if (!o_out) return KVLR_ERR_INVALID_ARGUMENT;
  return decode_attn_impl(shape, factors, cache, q, q_proj, seq_lens, page_table,
                          max_pages_per_seq, sel_pages, sel_phys, sel_counts, k_max, softmax_scale,
                          z_out, lse_out, o_out, nullptr, 0, batch, stream, true);
}

size_t kvlr_noalloc_scratch_bytes(void) { return kStaticScratchBytes; }

kvlr_status kvlr_upproject(const kvlr_shape* shape, const kvlr_factors* factors, const float* z,
                           float* o_out, int32_t batch, void* stream) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  if (!factors || batch < 0) return KVLR_ERR_INVALID_ARGUMENT;
  if (batch == 0) return KVLR_OK;
  if (!ok_ptr(factors->B_v) || !ok_ptr(z) || !ok_ptr(o_out)) return KVLR_ERR_INVALID_ARGUMENT;
  kvlr::UpprojArgs a{};
  a.dm = dm;
  a.B_v = factors->B_v;
  a.z = z;
  a.o = o_out;
  a.batch = batch;
  return hip_status(kvlr::launch_upproject(a, as_stream(stream)));
}

kvlr_status kvlr_fold_output_weights(const kvlr_shape* shape, const kvlr_factors* factors,
                                     const void* W_o, int32_t hidden, void* F_out, void* stream) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  if (dm.dtype != KVLR_DTYPE_BF16) return KVLR_ERR_UNSUPPORTED;
  if (!factors || hidden < 16 || hidden % 16 != 0 || hidden > (1 << 20)) return KVLR_ERR_INVALID_ARGUMENT;
  if (!ok_ptr(factors->B_v) || !ok_ptr(W_o) || !ok_ptr(F_out)) return KVLR_ERR_INVALID_ARGUMENT;
  kvlr::FoldArgs a{};
  a.dm = dm;
  a.W_o = W_o;
  a.B_v = factors->B_v;
  a.F = F_out;
  a.hidden = hidden;
  return hip_status(kvlr::launch_fold(a, as_stream(stream)));
}

kvlr_status kvlr_output_projection(const kvlr_shape* shape, const void* F, const float* z,
                                   int32_t hidden, float* out, int32_t batch, void* stream) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  if (dm.dtype != KVLR_DTYPE_BF16) return KVLR_ERR_UNSUPPORTED;
  if (batch < 0 || hidden < 16 || hidden % 16 != 0 || hidden > (1 << 20)) return KVLR_ERR_INVALID_ARGUMENT;
  if (batch == 0) return KVLR_OK;
  if (!ok_ptr(F) || !ok_ptr(z) || !ok_ptr(out)) return KVLR_ERR_INVALID_ARGUMENT;
  kvlr::OprojArgs a{};
  a.dm = dm;
  a.F = F;
  a.z = z;
  a.out = out;
  a.hidden = hidden;
  a.batch = batch;
  return hip_status(kvlr::launch_oproj(a, as_stream(stream)));
}

size_t kvlr_fit_workspace_bytes(const kvlr_shape* shape, int32_t n) {
  Dims dm;
  if (check_shape(shape, &dm) != KVLR_OK || n < 0) return 0;
  const size_t per_run = static_cast<size_t>(dm.Hkv) * 3 * dm.D * dm.D;
  const int runs = n > 0 ? kvlr::fit_runs(dm.Hkv, n).runs : 0;
  return round_up(per_run * sizeof(double)) + round_up(runs * per_run * sizeof(float));
}

kvlr_status kvlr_fit_moments(const kvlr_shape* shape, const void* k, const void* v, int32_t n,
                             double* moments, int32_t accumulate, void* workspace, size_t ws_bytes,
                             void* stream) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  if (n < 0 || (accumulate != 0 && accumulate != 1) || !ok_ptr(moments)) return KVLR_ERR_INVALID_ARGUMENT;
  if (n > 0 && (!ok_ptr(k) || !ok_ptr(v) || !ok_ptr(workspace))) return KVLR_ERR_INVALID_ARGUMENT;
  if (ws_bytes < kvlr_fit_workspace_bytes(shape, n)) return KVLR_ERR_WORKSPACE_TOO_SMALL;
  const size_t per_run = static_cast<size_t>(dm.Hkv) * 3 * dm.D * dm.D;
  kvlr::FitArgs a{};
  a.dm = dm;
  a.k = k;
  a.v = v;
  a.n = n;
  a.partial = n > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                               round_up(per_run * sizeof(double)))
                    : nullptr;
  a.moments = moments;
  a.accumulate = accumulate;
  return hip_status(kvlr::launch_fit_moments(a, as_stream(stream)));
}

// Joint decoder fit: sizes and buffers. nl = H_q rank_v latents per sample,
// nx = H_q head_dim outputs per sample.
static bool joint_dims(const Dims& dm, long* nl, long* nx) {
  *nl = static_cast<long>(dm.Hq) * dm.RV;
  *nx = static_cast<long>(dm.Hq) * dm.D;
  return *nl <= 4096 && *nx <= 16384;
}

size_t kvlr_fit_joint_workspace_bytes(const kvlr_shape* shape, int32_t n) {
  Dims dm;
  long nl = 0, nx = 0;
  if (check_shape(shape, &dm) != KVLR_OK || n < 0 || dm.lat == 2 || !joint_dims(dm, &nl, &nx)) return 0;
  return round_up(static_cast<size_t>(n) * nl * sizeof(float)) +        // latent outputs Z
         round_up(static_cast<size_t>(nl) * nl * sizeof(double)) +      // Z^T Z
         round_up(static_cast<size_t>(nl) * nx * sizeof(double)) +      // Z^T X
         round_up(static_cast<size_t>(nl) * nx * sizeof(float));        // decoder for the fold
}

kvlr_status kvlr_fit_joint_moments(const kvlr_shape* shape, const kvlr_factors* factors,
                                   const float* x, int32_t n, double* zz, double* zx,
                                   int32_t accumulate, void* workspace, size_t ws_bytes,
                                   void* stream) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  long nl = 0, nx = 0;
  if (dm.lat == 2 || !joint_dims(dm, &nl, &nx)) return KVLR_ERR_UNSUPPORTED;
  if (!factors || n < 0 || (accumulate != 0 && accumulate != 1) || !ok_ptr(zz) || !ok_ptr(zx))
    return KVLR_ERR_INVALID_ARGUMENT;
  if (n > 0 && (!ok_ptr(factors->A_v) || !ok_ptr(x) || !ok_ptr(workspace)))
    return KVLR_ERR_INVALID_ARGUMENT;
  if (n > 0 && ws_bytes < round_up(static_cast<size_t>(n) * nl * sizeof(float)))
    return KVLR_ERR_WORKSPACE_TOO_SMALL;
  kvlr::JointArgs a{};
  a.dm = dm;
  a.A_v = factors->A_v;
  a.x = x;
  a.n = n;
  a.z = static_cast<float*>(workspace);
  a.zz = zz;
  a.zx = zx;
  a.accumulate = accumulate;
  if (n == 0) {
    if (accumulate) return KVLR_OK;
    hipError_t e = kvlr::launch_zero_fill(zz, static_cast<size_t>(nl) * nl * sizeof(double), as_stream(stream));
    if (e == hipSuccess)
      e = kvlr::launch_zero_fill(zx, static_cast<size_t>(nl) * nx * sizeof(double), as_stream(stream));
    return hip_status(e);
  }
  return hip_status(kvlr::launch_joint_moments(a, as_stream(stream)));
}

kvlr_status kvlr_fit_joint_solve(const kvlr_shape* shape, const double* zz, const double* zx,
                                 double* D_out) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  long nl = 0, nx = 0;
  if (dm.lat == 2 || !joint_dims(dm, &nl, &nx)) return KVLR_ERR_UNSUPPORTED;
  if (!zz || !zx || !D_out) return KVLR_ERR_INVALID_ARGUMENT;
  return kvlr::joint_solve(static_cast<int>(nl), static_cast<int>(nx), zz, zx, D_out) == kvlr::FitStatus::kOk
             ? KVLR_OK
             : KVLR_ERR_NUMERICAL;
}

kvlr_status kvlr_fold_joint_decoder(const kvlr_shape* shape, const void* W_o, int32_t hidden,
                                    const float* D, void* F_out, void* stream) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  long nl = 0, nx = 0;
  if (dm.dtype != KVLR_DTYPE_BF16 || dm.lat == 2 || !joint_dims(dm, &nl, &nx)) return KVLR_ERR_UNSUPPORTED;
  if (hidden < 1 || hidden > (1 << 20) || !ok_ptr(W_o) || !ok_ptr(D) || !ok_ptr(F_out))
    return KVLR_ERR_INVALID_ARGUMENT;
  kvlr::JointFoldArgs a{};
  a.dm = dm;
  a.W_o = W_o;
  a.Dm = D;
  a.F = F_out;
  a.hidden = hidden;
  return hip_status(kvlr::launch_joint_fold(a, as_stream(stream)));
}

kvlr_status kvlr_choose_residual_ranks(const kvlr_shape* shape, const double* lam_k,
                                       double energy_frac, int32_t* ranks_out) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  if (!dm.exact) return KVLR_ERR_UNSUPPORTED;
  if (!lam_k || !ranks_out || !(energy_frac > 0.0) || energy_frac > 1.0) return KVLR_ERR_INVALID_ARGUMENT;
  for (int g = 0; g < dm.Hkv; ++g) {
    const double* lam = lam_k + static_cast<size_t>(g) * dm.RK;
    double total = 0.0;
    for (int i = 0; i < dm.RK; ++i) total += lam[i] > 0.0 ? lam[i] : 0.0;
    int pick = dm.RK;
    double run = 0.0;
    int i = 0;
    for (int r = 16; r <= dm.RK; r *= 2) {
      for (; i < r; ++i) run += lam[i] > 0.0 ? lam[i] : 0.0;
      if (run >= energy_frac * total) {
        pick = r;
        break;
      }
    }
    ranks_out[g] = pick;
  }
  return KVLR_OK;
}

kvlr_status kvlr_fit_solve(const kvlr_shape* shape, const double* moments, double* A_v,
                           double* A_k, double* W_pred, double* lam_v, double* lam_k) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  if (!moments || !A_v || !A_k || (dm.exact && !W_pred)) return KVLR_ERR_INVALID_ARGUMENT;
  const kvlr::FitStatus fs = kvlr::fit_solve(dm, moments, A_v, A_k, W_pred, lam_v, lam_k);
  return fs == kvlr::FitStatus::kOk ? KVLR_OK : KVLR_ERR_NUMERICAL;
}

}  // extern "C"

namespace {

uint16_t bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// host image of a float64 matrix in the storage type; transposed from
// [H][rows][cols] to [H][cols][rows] when asked
std::vector<uint8_t> storage_image(const std::vector<double>& m, int H, int rows, int cols,
                                   bool transpose, int dtype) {
  const size_t elem = dtype == KVLR_DTYPE_BF16 ? 2 : 4;
  std::vector<uint8_t> out(m.size() * elem);
  for (int g = 0; g < H; ++g)
    for (int i = 0; i < rows; ++i)
      for (int j = 0; j < cols; ++j) {
        const size_t src = (static_cast<size_t>(g) * rows + i) * cols + j;
        const size_t dst = transpose ? (static_cast<size_t>(g) * cols + j) * rows + i : src;
        const float f = static_cast<float>(m[src]);
        if (elem == 2) {
          const uint16_t b = bf16_rne(f);
          memcpy(&out[dst * 2], &b, 2);
        } else {
          memcpy(&out[dst * 4], &f, 4);
        }
      }
  return out;
}

}  // namespace

extern "C" {

kvlr_status kvlr_fit_factors(const kvlr_shape* shape, const void* k, const void* v, int32_t n,
                             const kvlr_factor_buffers* out, double* lam_v, double* lam_k,
                             void* workspace, size_t ws_bytes, void* stream) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  if (n < 1 || !out || !ok_ptr(out->A_v) || !ok_ptr(out->B_v) || !ok_ptr(out->A_k) ||
      !ok_ptr(out->B_k) || (dm.exact && !ok_ptr(out->W_pred)) || !ok_ptr(workspace))
    return KVLR_ERR_INVALID_ARGUMENT;
  if (ws_bytes < kvlr_fit_workspace_bytes(shape, n)) return KVLR_ERR_WORKSPACE_TOO_SMALL;
  double* moments = static_cast<double*>(workspace);
  st = kvlr_fit_moments(shape, k, v, n, moments, 0, workspace, ws_bytes, stream);
  if (st != KVLR_OK) return st;
  const hipStream_t s = as_stream(stream);
  const int H = dm.Hkv, D = dm.D, RV = dm.RV, RK = dm.RK;
  std::vector<double> mom(static_cast<size_t>(H) * 3 * D * D);
  hipError_t e = hipMemcpyAsync(mom.data(), moments, mom.size() * sizeof(double),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e);
  std::vector<double> A_v(static_cast<size_t>(H) * D * RV), A_k(static_cast<size_t>(H) * D * RK),
      W(dm.exact ? static_cast<size_t>(H) * RV * D : 0);
  if (kvlr::fit_solve(dm, mom.data(), A_v.data(), A_k.data(), dm.exact ? W.data() : nullptr, lam_v,
                      lam_k) != kvlr::FitStatus::kOk)
    return KVLR_ERR_NUMERICAL;
  struct Item {
    void* dst;
    std::vector<uint8_t> img;
  };
  std::vector<Item> items;
  items.push_back({out->A_v, storage_image(A_v, H, D, RV, false, dm.dtype)});
  items.push_back({out->B_v, storage_image(A_v, H, D, RV, true, dm.dtype)});
  items.push_back({out->A_k, storage_image(A_k, H, D, RK, false, dm.dtype)});
  items.push_back({out->B_k, storage_image(A_k, H, D, RK, true, dm.dtype)});
  if (dm.exact) items.push_back({out->W_pred, storage_image(W, H, RV, D, false, dm.dtype)});
  for (auto& it : items) {
    e = hipMemcpyAsync(it.dst, it.img.data(), it.img.size(), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_status(e);
  }
  return hip_status(hipStreamSynchronize(s));  // the host images must outlive the copies
}

kvlr_status kvlr_fit_joint(const kvlr_shape* shape, const kvlr_factors* factors, const float* x,
                           int32_t n, const void* W_o, int32_t hidden, void* F_out, double* D_out,
                           void* workspace, size_t ws_bytes, void* stream) {
  Dims dm;
  kvlr_status st = check_shape(shape, &dm);
  if (st != KVLR_OK) return st;
  long nl = 0, nx = 0;
  if (dm.dtype != KVLR_DTYPE_BF16 || dm.lat == 2 || !joint_dims(dm, &nl, &nx)) return KVLR_ERR_UNSUPPORTED;
  if (n < 1 || hidden < 1 || hidden > (1 << 20) || !factors || !ok_ptr(factors->A_v) || !ok_ptr(x) ||
      !ok_ptr(W_o) || !ok_ptr(F_out) || !ok_ptr(workspace))
    return KVLR_ERR_INVALID_ARGUMENT;
  if (ws_bytes < kvlr_fit_joint_workspace_bytes(shape, n)) return KVLR_ERR_WORKSPACE_TOO_SMALL;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const size_t oz = round_up(static_cast<size_t>(n) * nl * sizeof(float));
  const size_t ozz = oz + round_up(static_cast<size_t>(nl) * nl * sizeof(double));
  const size_t ozx = ozz + round_up(static_cast<size_t>(nl) * nx * sizeof(double));
  double* zz = reinterpret_cast<double*>(ws + oz);
  double* zx = reinterpret_cast<double*>(ws + ozz);
  float* Dm = reinterpret_cast<float*>(ws + ozx);
  st = kvlr_fit_joint_moments(shape, factors, x, n, zz, zx, 0, workspace, ws_bytes, stream);
  if (st != KVLR_OK) return st;
  const hipStream_t s = as_stream(stream);
  std::vector<double> hzz(static_cast<size_t>(nl) * nl), hzx(static_cast<size_t>(nl) * nx),
      hD(static_cast<size_t>(nl) * nx);
  hipError_t e = hipMemcpyAsync(hzz.data(), zz, hzz.size() * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(hzx.data(), zx, hzx.size() * sizeof(double), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e);
  if (kvlr::joint_solve(static_cast<int>(nl), static_cast<int>(nx), hzz.data(), hzx.data(), hD.data()) !=
      kvlr::FitStatus::kOk)
    return KVLR_ERR_NUMERICAL;
  if (D_out) memcpy(D_out, hD.data(), hD.size() * sizeof(double));
  std::vector<float> hDf(hD.size());
  for (size_t i = 0; i < hD.size(); ++i) hDf[i] = static_cast<float>(hD[i]);
  e = hipMemcpyAsync(Dm, hDf.data(), hDf.size() * sizeof(float), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_status(e);
  st = kvlr_fold_joint_decoder(shape, W_o, hidden, Dm, F_out, stream);
  if (st != KVLR_OK) return st;
  return hip_status(hipStreamSynchronize(s));  // the host copy of D must outlive the upload
}

}  // extern "C"
