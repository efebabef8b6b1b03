// Host-side launch interfaces between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvlr_host.h"

namespace kvlr {

// Shape facts every launcher needs, already validated by the API layer.
struct Dims {
  int Hq, Hkv, G, D, P, RV, RK;
  int dtype;      // factors, original keys, new tokens: 0 bf16, 1 f32
  int lat;        // latents (v_lat, k_lat): 0 bf16, 1 f32, 2 FP8 E4M3
  int exact;      // 1 = routed (residual latent + original keys)
};

// Residual-latent (k_lat) layout of a routed cache. Uniform: every KV head
// keeps rank_k / CH chunk columns, head g at chunk offset g * that. Adaptive
// (per-head residual ranks): head g keeps ck[g] chunk columns at chunk offset
// off[g] of its page, and a page holds page_chunks chunk columns in all.
constexpr int kMaxAdaptiveHeads = 16;
struct KLayout {
  int adaptive;
  int page_chunks;
  int ck[kMaxAdaptiveHeads];
  int off[kMaxAdaptiveHeads];
  int rpc[kMaxAdaptiveHeads];  // routing rows per work chunk of head g (equal bytes per chunk)
};

struct QprojArgs {
  Dims dm;
  const void* W_pred;  // [Hkv][RV][D] (exact only)
  const void* B_k;     // [Hkv][RK][D]
  const float* q;      // [B][Hq][D]
  float* q_proj;       // [B][Hq][width]
  int batch;
};
hipError_t launch_qproj(const QprojArgs& a, hipStream_t s);

struct RouteArgs {
  Dims dm;
  const void* v_lat;
  const void* k_lat;
  const float* q_proj;
  const int32_t* seq_lens;
  const int32_t* page_table;
  int max_pages;
  int topk_num, topk_den, k_max;
  const int32_t* k_pages;  // optional [B]: pages kept per sequence (else the fraction)
  int32_t* sel;
  int32_t* sel_counts;  // optional [B][Hkv]
  int32_t* sel_phys;    // optional [B][Hkv][k_max]: physical pages of sel
  float* scores;        // [B][Hkv][max_pages]
  uint32_t* counters;   // [B * Hkv], zero between calls
  KLayout kl;
  int batch;
  int rows_per_chunk;   // 64-token rows per work chunk
  int static_splits;    // > 0: chunks per pair fixed from the table width (no pass over the lengths);
                        // with per-head ranks, the table's rows (each head splits them itself)
  int scores_only;      // 1: page scores only, no selection launch (sel outputs unused)
  int grid;             // persistent workgroups
};
hipError_t launch_route(const RouteArgs& a, hipStream_t s);
hipError_t launch_select(const RouteArgs& a, hipStream_t s);  // selection alone, from a.scores
int route_rows_per_chunk(int row_bytes);  // row_bytes: one 64-token row of [v | c] latents

struct AttnArgs {
  Dims dm;
  const void* keys;      // k_exact (exact) or k_lat (latent)
  const void* v_lat;
  const float* qsrc;     // q (exact) or q_proj (latent)
  int q_stride;          // floats per (b, h) row of qsrc
  const int32_t* seq_lens;
  const int32_t* page_table;
  int max_pages;
  const int32_t* sel;    // NULL = every page
  const int32_t* sel_phys;    // optional physical pages of sel
  const int32_t* sel_counts;  // optional valid entries per (sequence, KV head)
  int k_max;
  float scale_log2e;
  float* partials;       // [B*Hkv][num_splits][G][RV + 2]
  float* z_out;
  float* lse_out;        // may be NULL
  const void* B_v;       // with o_out: up-project z in the merge launch
  float* o_out;          // may be NULL
  int batch;
  int rows_per_chunk;    // 64-token rows per work chunk
  int max_splits;        // chunk slots per pair in the partials buffer
  int grid;              // persistent workgroups
};
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);
int attn_rows_per_chunk(bool selected);

struct UpprojArgs {
  Dims dm;
  const void* B_v;
  const float* z;
  float* o;
  int batch;
};
hipError_t launch_upproject(const UpprojArgs& a, hipStream_t s);

struct FoldArgs {
  Dims dm;
  const void* W_o;  // [hidden][Hq * D] bf16
  const void* B_v;  // [Hkv][RV][D] bf16
  void* F;          // [hidden][Hq * RV] bf16
  int hidden;
};
hipError_t launch_fold(const FoldArgs& a, hipStream_t s);

struct OprojArgs {
  Dims dm;
  const void* F;    // [hidden][Hq * RV] bf16
  const float* z;   // [B][Hq][RV]
  float* out;       // [B][hidden]
  int hidden;
  int batch;
};
hipError_t launch_oproj(const OprojArgs& a, hipStream_t s);

struct EncodeArgs {
  Dims dm;
  const void* A_v;
  const void* A_k;
  const void* W_pred;
  const void* k_new;
  const void* v_new;
  const int32_t* cu_new;
  const int32_t* lens_before;
  const int32_t* page_table;
  int max_pages;
  void* v_lat;
  void* k_lat;
  void* k_exact;
  int batch;
  int total_new;
  KLayout kl;
  // optional: the step's query images from the same launch (q NULL: none)
  const void* B_k;      // [Hkv][RK][D]
  const float* q;       // [B][Hq][D]
  float* q_proj;        // [B][Hq][width]
  // optional (exact keys): -W_pred A_k prepared by launch_encode_prep
  const void* m_prep;
};
hipError_t launch_encode(const EncodeArgs& a, hipStream_t s);
// Writes -W_pred A_k per KV head in the encode's operand layout (exact keys;
// reads a.dm, a.A_k, a.W_pred, a.kl); encode_prep_bytes: its size, 0 if the
// shape has none or is not supported.
hipError_t launch_encode_prep(const EncodeArgs& a, void* out, hipStream_t s);
size_t encode_prep_bytes(const Dims& dm);

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s);
// errors[0] |= 1 for a table entry in use outside [0, num_phys), 2 for a length
// outside [0, max_pages * P]; errors[1] = bad entries (both cleared first)
hipError_t launch_check_tables(const int32_t* seq_lens, const int32_t* page_table, int max_pages,
                               int P, int num_phys, int batch, uint32_t* errors, hipStream_t s);

// Factor fitting: second moments of sample keys and values per KV head.
struct FitArgs {
  Dims dm;
  const void* k;      // [n][Hkv][D] samples, storage type
  const void* v;
  int n;
  float* partial;     // [runs][Hkv][3][D][D] per-run float32 sums
  double* moments;    // [Hkv][3][D][D]: V^T V, K^T K, V^T K
  int accumulate;     // add onto moments instead of overwriting
};
struct FitRuns {
  int runs;   // token runs (workgroups per KV head)
  int chunk;  // tokens per run, a multiple of 64
};
FitRuns fit_runs(int Hkv, int n);
hipError_t launch_fit_moments(const FitArgs& a, hipStream_t s);

// Host: factors from float64 moments. A_v [Hkv][D][RV], A_k [Hkv][D][RK],
// W [Hkv][RV][D] (exact keys only), lam_v [Hkv][RV], lam_k [Hkv][RK] (may
// be null).
FitStatus fit_solve(const Dims& dm, const double* moments, double* A_v, double* A_k, double* W,
                    double* lam_v, double* lam_k);

// Joint decoder fit: latent outputs Z = X A per head and the moments Z^T Z,
// Z^T X (float64), then the fold F = W_o D^T of a decoder D.
struct JointArgs {
  Dims dm;
  const void* A_v;  // [Hkv][D][RV] storage type
  const float* x;   // [n][Hq][D] attention outputs
  int n;
  float* z;         // [n][Hq RV] workspace
  double* zz;       // [Hq RV][Hq RV]
  double* zx;       // [Hq RV][Hq D]
  int accumulate;   // add onto zz, zx
};
hipError_t launch_joint_moments(const JointArgs& a, hipStream_t s);
struct JointFoldArgs {
  Dims dm;
  const void* W_o;  // [hidden][Hq D] bf16
  const float* Dm;  // [Hq RV][Hq D] decoder
  void* F;          // [hidden][Hq RV] bf16
  int hidden;
};
hipError_t launch_joint_fold(const JointFoldArgs& a, hipStream_t s);


}  // namespace kvlr
