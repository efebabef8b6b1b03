// Page routing for the routed (exact-key) cache.
//
// BasisKV: Value Latents for Communication and Key Routing, English abstract:
// the stored value latent predicts part of each key, a key-specific residual
// latent holds the rest, and the two together decide which key pages are
// read. In latent space the approximate score of token t for query head h is
//   s[h, t] = q_hat_h . v_t + q_tilde_h . c_t,
// q_hat = q W_pred^T and q_tilde = q B_k^T (computed once per step by the
// query-projection kernel). A page's score is the max over its valid tokens
// and the KV group's heads; the k_b best pages are kept.
//
// Work split: one lane per token. A 64-token "row" of one (sequence, KV head)
// pair is read with 16-byte loads; the page layout puts the P tokens of one
// 16-byte chunk column next to each other, so a wave's load of one chunk
// column is one contiguous run. The projected queries are wave-uniform and
// are read with scalar loads. Each workgroup (4 waves) scores a range of rows;
// the last workgroup of a pair to finish (an atomic ticket) runs the exact
// top-k for the pair: a 4-pass radix select on order-preserving 32-bit keys
// followed by an ascending ballot compaction.

#include "kvlr_device.h"
#include "kvlr_internal.h"
#include "kvlr_select.h"

#ifndef KVLR_ROUTE_ROLLING
#define KVLR_ROUTE_ROLLING 1
#endif
#ifndef KVLR_ROUTE_MFMA
#define KVLR_ROUTE_MFMA 1
#endif


namespace kvlr {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;


// Exclusive prefix count of `flag` over the workgroup in thread order; also
// returns the total. Uses one LDS slot per wave; contains two barriers.
__device__ inline int block_excl_count(bool flag, int* total, int* lds4) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const uint64_t m = __ballot(flag);
  const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) lds4[wave] = __popcll(m);
  __syncthreads();
  int before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = lds4[w];
    before += (w < wave) ? c : 0;
    sum += c;
  }
  __syncthreads();
  *total = sum;
  return before + in_wave;
}

// Top-k of scores[0..N) into sel[0..k_max): k largest, ties to the lower
// index, ascending, -1 padding; with sel_phys, also each chosen page's
// physical page pt[j] (-1 padding). Also writes -inf to scores[N..max_pages).
__device__ void select_pages(float* scores, int N, int k, int k_max, int max_pages, int32_t* sel,
                             const int32_t* pt, int32_t* sel_phys) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_digit;
  __shared__ int s_kk;
  __shared__ int lds4[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);

  const bool take_all = (k >= N);
  uint32_t prefix = 0, pmask = 0;
  int kk = k;
  if (!take_all && k > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;  // kThreads == 256 bins
      __syncthreads();
      for (int j = tid; j < N; j += kThreads) {
        const uint32_t key = order_key(load_shared_f32(&scores[j]));
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < kWave) {
        // lane l owns bins 4l .. 4l+3; suffix sums from the top bin down
        const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
        const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
        const uint32_t local = h0 + h1 + h2 + h3;
        uint32_t suf = local;  // sum over lanes >= lane
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const uint32_t o = __shfl_down(suf, off, kWave);
          if (lane + off < kWave) suf += o;
        }
        const uint64_t hit = __ballot(suf >= static_cast<uint32_t>(kk));
        const int top = 63 - __clzll(hit);  // highest lane whose suffix reaches kk
        if (lane == top) {
          uint32_t above = suf - local;  // count in bins above this lane's
          const uint32_t hs[4] = {h0, h1, h2, h3};
          int d = 3;
          for (; d > 0; --d) {
            if (above + hs[d] >= static_cast<uint32_t>(kk)) break;
            above += hs[d];
          }
          s_digit = static_cast<uint32_t>(4 * lane + d);
          s_kk = kk - static_cast<int>(above);
        }
      }
      __syncthreads();
      prefix |= s_digit << shift;
      pmask |= 255u << shift;
      kk = s_kk;
      __syncthreads();
    }
  }
  // prefix = key of the k-th largest score; kk = how many of the equal keys to take
  int taken = 0, eq_seen = 0;
  for (int j0 = 0; j0 < N; j0 += kThreads) {
    const int j = j0 + tid;
    const bool in = j < N;
    const uint32_t key = in ? order_key(load_shared_f32(&scores[j])) : 0u;
    const bool gt = in && (take_all || key > prefix);
    const bool eq = in && !take_all && k > 0 && key == prefix;
    int eq_total = 0;
    const int eq_rank = eq_seen + block_excl_count(eq, &eq_total, lds4);
    const bool take = gt || (eq && eq_rank < kk);
    int take_total = 0;
    const int pos = taken + block_excl_count(take, &take_total, lds4);
    if (take && pos < k_max) {
      sel[pos] = j;
      if (sel_phys) sel_phys[pos] = pt[j];
    }
    taken += take_total;
    eq_seen += eq_total;
  }
  for (int i = k + tid; i < k_max; i += kThreads) {
    sel[i] = -1;
    if (sel_phys) sel_phys[i] = -1;
  }
  for (int j = N + tid; j < max_pages; j += kThreads) scores[j] = -__builtin_huge_valf();
}

// select_pages for N <= kSelectLds: the order keys are read once into LDS and
// selected there (select_keys_lds). With sel_phys, the sequence's page-table
// row is read into LDS together with the scores (no extra wait), and each
// chosen page's physical page is written too.
__device__ void select_pages_lds(float* scores, int N, int k, int k_max, int max_pages,
                                 int32_t* sel, const int32_t* pt, int32_t* sel_phys) {
  __shared__ SelectLds s;
  const int tid = threadIdx.x;
  // The scores are read with coherent device-scope loads through a global
  // (not generic) pointer, eight per thread at a time, all issued before the
  // first is used: one at a time, each would wait out a full memory latency.
  // Indices past N re-read score N-1 and are not kept.
  typedef __attribute__((address_space(1))) float gfloat;
  gfloat* gs = (gfloat*)scores;
  select_lds_clear(s);
  for (int j0 = 0; j0 < N; j0 += 8 * kThreads) {
    float v[8];
    int32_t ph[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = min(j0 + u * kThreads + tid, N - 1);
      v[u] = __hip_atomic_load(gs + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (sel_phys) ph[u] = pt[j];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u * kThreads + tid;
      if (j < N) {
        s.keys[j] = order_key(v[u]);
        if (sel_phys) s.pt[j] = ph[u];
      }
    }
  }
  __syncthreads();
  select_keys_lds<kThreads>(s, N, k, [&](int pos, int j) {
    if (pos < k_max) {
      sel[pos] = j;
      if (sel_phys) sel_phys[pos] = s.pt[j];
    }
  });
  for (int i = k + tid; i < k_max; i += kThreads) {
    sel[i] = -1;
    if (sel_phys) sel_phys[i] = -1;
  }
  for (int j = N + tid; j < max_pages; j += kThreads) scores[j] = -__builtin_huge_valf();
}

__device__ inline void select_top_pages(float* scores, int N, int k, int k_max, int max_pages,
                                        int32_t* sel, const int32_t* pt, int32_t* sel_phys) {
  if (N <= kSelectLds)
    select_pages_lds(scores, N, k, k_max, max_pages, sel, pt, sel_phys);
  else
    select_pages(scores, N, k, k_max, max_pages, sel, pt, sel_phys);
}

// Top-k selection of each (sequence, KV head) pair from the page scores the
// routing launch wrote (one workgroup per pair, in a launch of its own after
// the scores). Against selecting in the routing launch's last workgroup of
// each pair, no routing workgroup waits for its score stores or takes a
// ticket, and the selections run side by side once every score is written.
// NT = 1024 serves tables of 1025 .. kSelectLds pages and NT = 512 tables of
// 257 .. 1024 (keys in LDS, at most two per thread); NT = 256 any count.
template <int NT>
__global__ __launch_bounds__(NT) void select_kernel(
    float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ page_table, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_counts, int32_t* __restrict__ sel_phys,
    const int32_t* __restrict__ k_pages, int Hkv, int P, int log2P, int max_pages, int topk_num,
    int topk_den, int k_max) {
  const int pair = blockIdx.x;
  const int b = pair / Hkv;
  const int L = table_len(seq_lens[b], max_pages, P);
  const int N = (L + P - 1) >> log2P;
  const int k = pages_to_keep(N, k_pages, b, topk_num, topk_den, k_max);
  float* sc = scores + static_cast<size_t>(pair) * max_pages;
  int32_t* so = sel + static_cast<size_t>(pair) * k_max;
  int32_t* spo = sel_phys ? sel_phys + static_cast<size_t>(pair) * k_max : nullptr;
  const int32_t* pt = page_table + static_cast<size_t>(b) * max_pages;
  if constexpr (NT == kThreads) {
    select_top_pages(sc, N, k, k_max, max_pages, so, pt, spo);
  } else {
    // N <= kSelectLds (the host picks NT = 1024 only then): every key and
    // table entry requested at once, then the selection in LDS
    __shared__ SelectLds s;
    const int tid = threadIdx.x;
    constexpr int PER = NT == 512 ? 2 : kSelectLds / NT;  // NT = 512: at most 1024 pages
    float v[PER];
    int32_t ph[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int j = min(u * NT + tid, max(N - 1, 0));
      v[u] = sc[j];
      ph[u] = spo ? pt[j] : 0;
    }
    select_lds_clear(s);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int j = u * NT + tid;
      if (j < N) {
        s.keys[j] = order_key(v[u]);
        s.pt[j] = ph[u];
      }
    }
    __syncthreads();
    select_keys_lds<NT>(s, N, k, [&](int pos, int j) {
      if (pos < k_max) {
        so[pos] = j;
        if (spo) spo[pos] = s.pt[j];
      }
    });
    for (int i = k + tid; i < k_max; i += NT) {
      so[i] = -1;
      if (spo) spo[i] = -1;
    }
    for (int j = N + tid; j < max_pages; j += NT) sc[j] = -__builtin_huge_valf();
  }
  if (threadIdx.x == 0 && sel_counts) sel_counts[pair] = k;
}

// Scores of one 64-token row: acc[h] = q_hat_h . v + q_tilde_h . c per lane,
// the group's projected queries broadcast from VGPRs (NQ = G*W/16).
template <class S, int G, int RV, int RK, int NQ>
__device__ inline float row_score(const float (&qv)[NQ], const uint4 (&vc)[RV / S::CH],
                                  const uint4 (&kc)[RK / S::CH]) {
  constexpr int CH = S::CH, CV = RV / CH, CK = RK / CH, W = RV + RK;
  float acc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h] = 0.f;
  static_for<0, CV>([&](auto cc) {
    constexpr int C = decltype(cc)::value;
    float x[CH];
    S::unpack(vc[C], x);
    fma_heads_bcast<G, CH, W, C * CH>(qv, x, acc);
  });
  static_for<0, CK>([&](auto cc) {
    constexpr int C = decltype(cc)::value;
    float x[CH];
    S::unpack(kc[C], x);
    fma_heads_bcast<G, CH, W, RV + C * CH>(qv, x, acc);
  });
  float m = acc[0];
#pragma unroll
  for (int h = 1; h < G; ++h) m = fmaxf(m, acc[h]);
  return m;
}

// ROWPAGE: page_size == 64, so a row is exactly one page; its page-table
// entry and base address are wave-uniform, and the next row's loads are
// issued before the current row is scored.
// ADAPT: per-head residual ranks (the residual's chunk count and offset are
// per head); uniform caches keep them compile-time, so address offsets fold
// into the load instructions.
template <class S, int G, int RV, int RK, bool ROWPAGE, bool ADAPT = false>
#ifndef KVLR_ROUTE_WAVES_PER_EU
#define KVLR_ROUTE_WAVES_PER_EU 1  // the least waves per SIMD the registers must allow
#endif
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(KVLR_ROUTE_WAVES_PER_EU))) void route_kernel(
    const uint8_t* __restrict__ v_lat, const uint8_t* __restrict__ k_lat,
    const float* __restrict__ q_proj, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ page_table, float* __restrict__ scores,
    uint32_t* __restrict__ counters, int32_t* __restrict__ sel, int32_t* __restrict__ sel_counts,
    int32_t* __restrict__ sel_phys, const int32_t* __restrict__ k_pages, int Hq, int Hkv, int P,
    int log2P, int max_pages, int topk_num, int topk_den, int k_max, int rows_per_chunk,
    int static_splits, int scores_only, int batch, KLayout kl) {
  constexpr int CH = S::CH;
  constexpr int CV = RV / CH;
  constexpr int CK = RK / CH;
  constexpr int W = RV + RK;
  constexpr int NQ = G * W / 16;
  extern __shared__ int s_base[];
  __shared__ int s_last;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const size_t slab_v = static_cast<size_t>(CV) * P * S::CB;  // bytes of one head's page
  const size_t slab_k = static_cast<size_t>(CK) * P * S::CB;

  // work chunks of head g span rpc(g) rows: rows_per_chunk, or with per-head
  // residual ranks a count that gives every chunk about the same bytes
  auto rpc_of = [&](int g) { return ADAPT ? kl.rpc[g] : rows_per_chunk; };
  auto splits_of = [&](int rows, int g) { return max(1, (rows + rpc_of(g) - 1) / rpc_of(g)); };
  // With static_splits > 0 every pair has a fixed number of chunks, sized
  // for the longest row the page table allows (static_splits chunks; with
  // per-head ranks static_splits is the table's row count and each head
  // splits it by its own chunk size), and a chunk's pair and split follow
  // from its index alone: the sequence length, the projected queries and the
  // first rows' page-table entries are then requested together, with no pass
  // over the batch's lengths first. Chunks past a sequence's rows score
  // nothing.
  const bool fixed = static_splits > 0;
  int total, per_b = 0;
  if (fixed) {
    if constexpr (!ADAPT) {
      per_b = Hkv * static_splits;
    } else {
      for (int g = 0; g < Hkv; ++g) per_b += splits_of(static_splits, g);
    }
    total = batch * per_b;
  } else {
    build_chunk_prefix(batch, s_base, [&](int b) {
      const int rows = (table_len(seq_lens[b], max_pages, P) + kWave - 1) / kWave;
      if (!ADAPT) return Hkv * splits_of(rows, 0);
      int n = 0;
      for (int g = 0; g < Hkv; ++g) n += splits_of(rows, g);
      return n;
    });
    total = s_base[batch];
  }

  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    int b, local;
    if (fixed) {
      b = w / per_b;
      local = w - b * per_b;
    } else {
      b = __builtin_amdgcn_readfirstlane(find_sequence(s_base, batch, w));
      local = __builtin_amdgcn_readfirstlane(w - s_base[b]);
    }
    const int L = table_len(seq_lens[b], max_pages, P);
    const int nrows = (L + kWave - 1) / kWave;
    int g, nsplit;
    if (fixed && !ADAPT) {
      nsplit = static_splits;
      g = local / nsplit;
      local -= g * nsplit;
    } else if (!ADAPT) {
      nsplit = (s_base[b + 1] - s_base[b]) / Hkv;
      g = local / nsplit;
      local -= g * nsplit;
    } else {
      const int split_rows = fixed ? static_splits : nrows;
      g = 0;
      nsplit = splits_of(split_rows, 0);
      while (local >= nsplit) {
        local -= nsplit;
        nsplit = splits_of(split_rows, ++g);
      }
    }
    // every value here is the same across the workgroup; saying so keeps the
    // per-head table reads and what derives from them in scalar registers
    g = __builtin_amdgcn_readfirstlane(g);
    nsplit = __builtin_amdgcn_readfirstlane(nsplit);
    const int split = __builtin_amdgcn_readfirstlane(local);
    const int rpc = rpc_of(g);
    const int pair = b * Hkv + g;
    const float* __restrict__ qp = q_proj + static_cast<size_t>(b * Hq + g * G) * W;
    const int32_t* __restrict__ pt = page_table + static_cast<size_t>(b) * max_pages;
    float* __restrict__ sc = scores + static_cast<size_t>(pair) * max_pages;
    // the vector-ALU paths keep the projected queries spread over the lanes
    // (FP8 latents and per-head residual ranks have only the matrix-core path)
    constexpr bool kMfma = ROWPAGE && S::CH == 8 && (KVLR_ROUTE_MFMA || S::CB == 8 || ADAPT);
    float qv[kMfma ? 1 : NQ];
    if constexpr (!kMfma) load_q_rows(qp, qv);
    const int row0 = split * rpc;
    const int row1 = min(row0 + rpc, nrows);

    if constexpr (kMfma) {
      // Matrix-core scoring (bf16 or FP8 latents, one page per row). A 64-token
      // row is four 16-token tiles; per tile, scores[token][head] = sum over
      // the concatenated [v | c] latent (K, in steps of 32) of latent x query,
      // as v_mfma_f32_16x16x32_bf16 with tokens as rows (lane l: row l%16, 8
      // latent elements from k-group l/16: one chunk of the page) and heads as
      // columns (the projected queries split into bf16 high and low halves,
      // two products per step). A lane's 16-byte load holds TPL consecutive
      // tokens of one chunk column (1 bf16 chunk, or 2 FP8 chunks decoded
      // exactly to bf16), and tile t = p*TPL + h takes the tokens
      // TPL*(16p + row) + h, so one load feeds TPL tiles. Heads past the
      // group and tokens past the sequence end are masked before the page max.
      // k-steps: ceil(CV/4) over the value latent, then ceil(CK/4) over the
      // residual, so each step reads one slab (a uniform base address). With
      // per-head residual ranks this head's slab has ckg <= CK chunks at its
      // own offset; chunks past ckg are not read (their query half is zero).
      constexpr int KSV = (CV + 3) / 4, KSK = (CK + 3) / 4, KS = KSV + KSK;
      constexpr int TPL = 16 / S::CB;  // tokens per 16-byte load
      constexpr int NL = 4 / TPL;      // loads per k-step and row
      const int kq = lane >> 4, col = lane & 15;
      const int ckg = ADAPT ? kl.ck[g] : CK;
      const size_t kpage = ADAPT ? static_cast<size_t>(kl.page_chunks) * P * S::CB : Hkv * slab_k;
      const size_t koff = ADAPT ? static_cast<size_t>(kl.off[g]) * P * S::CB : g * slab_k;
      // Past the slab's last chunk a lane re-reads chunk 0 (its query half is
      // zero); past the last row every lane reads one shared address.
      struct RowRef {
        const uint8_t* vb;
        const uint8_t* kb;
        int on;  // 1 for a real row
      };
      // The entry is requested whether or not the row exists (an index within
      // the table row, clamped), so its request does not wait for the length;
      // a row past the chunk or the sequence reads page 0's slab at offset 0.
      auto row_ref = [&](int row) -> RowRef {
        const int ent = pt[min(row, max_pages - 1)];
        const bool on = row < row1;
        const size_t phys = on ? static_cast<size_t>(ent) : 0;
        return RowRef{v_lat + (phys * Hkv + g) * slab_v, k_lat + phys * kpage + koff, on ? 1 : 0};
      };
      auto a_addr = [&](const RowRef& rr, int p, int st) -> const uint8_t* {
        const bool on_v = st < KSV;
        int ci = 4 * (on_v ? st : st - KSV) + kq;
        if (ci >= (on_v ? CV : ckg)) ci = 0;
        const uint32_t off = static_cast<uint32_t>(rr.on) *
                             static_cast<uint32_t>(TPL * (p * 16 + col) * S::CB + ci * (kWave * S::CB));
        return (on_v ? rr.vb : rr.kb) + off;
      };
      int r = row0 + wave;
      uint4 A[NL][KS];
      // residual k-steps past this head's rank (per-head ranks) are skipped:
      // a wave-uniform test, compiled only where the residual spans 2+ steps
      const int ks_used = KSV + (ckg + 3) / 4;
      auto step_on = [&](int st) { return st <= KSV || st < ks_used; };
      // the projected queries are requested first, all k-steps at once (a
      // lane outside the group or past the slab reads the group's first row
      // and gets zeros), then the first row; their fragments are formed while
      // that row is in flight (the in-order counter lets them wait for the
      // queries alone)
      float4 qa[KS], qc[KS];
      bool qhave[KS];
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const bool on_v = st < KSV;
        const int ci = 4 * (on_v ? st : st - KSV) + kq;  // chunk within the slab
        qhave[st] = col < G && ci < (on_v ? CV : ckg);
        const float* src = qp + (qhave[st] ? col * W + (on_v ? 0 : RV) + ci * 8 : 0);
        qa[st] = *reinterpret_cast<const float4*>(src);
        qc[st] = *reinterpret_cast<const float4*>(src + 4);
      }
      RowRef cur = row_ref(r);
#pragma unroll
      for (int p = 0; p < NL; ++p)
#pragma unroll
        for (int st = 0; st < KS; ++st)
          if (step_on(st)) A[p][st] = load16_stream(a_addr(cur, p, st));
      RowRef nxt = row_ref(r + kWaves);
      bf16x8 qhi[KS], qlo[KS];
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        float x[8] = {qa[st].x, qa[st].y, qa[st].z, qa[st].w, qc[st].x, qc[st].y, qc[st].z, qc[st].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = qhave[st] ? x[e] : 0.f;
        split_bf16x8(x, qhi[st], qlo[st]);
      }
      for (; r < row1; r += kWaves) {
        const RowRef nn = row_ref(r + 2 * kWaves);  // page-table entry two rows ahead
        f32x4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < NL; ++p) {
#pragma unroll
          for (int st = 0; st < KS; ++st) {
            if (!step_on(st)) continue;
#pragma unroll
            for (int h = 0; h < TPL; ++h) {
              const bf16x8 a = S::frag_of16(A[p][st], h);
              f32x4& c = acc[p * TPL + h];
              c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qhi[st], c, 0, 0, 0);
              c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qlo[st], c, 0, 0, 0);
            }
            A[p][st] = load16_stream(a_addr(nxt, p, st));
          }
        }
        const int nvalid = L - r * kWave;
        float m = -__builtin_huge_valf();
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            // output row 4*kq + v of tile t is token TPL*(16*(t/TPL) + 4*kq + v) + t%TPL
            const int tok = TPL * (16 * (t / TPL) + 4 * kq + v) + t % TPL;
            const bool ok = col < G && tok < nvalid;
            m = ok ? fmaxf(m, acc[t][v]) : m;
          }
        m = wave_max_u(m);
        if (lane == 0) store_shared_f32(&sc[r], m);
        nxt = nn;
      }
    } else if constexpr (ROWPAGE) {
      // one page per row: its page-table entry and base address are uniform
      auto row_base = [&](int row, const uint8_t*& vbase, const uint8_t*& kbase) -> bool {
        const size_t phys = static_cast<size_t>(pt[row]);
        vbase = v_lat + (phys * Hkv + g) * slab_v + lane * 16;
        kbase = k_lat + (phys * Hkv + g) * slab_k + lane * 16;
        return lane < L - row * kWave;
      };
      auto finish_row = [&](int row, float (&acc)[G]) {
        float m = acc[0];
#pragma unroll
        for (int h = 1; h < G; ++h) m = fmaxf(m, acc[h]);
        if (lane >= L - row * kWave) m = -__builtin_huge_valf();
        m = wave_max_u(m);
        if (lane == 0) store_shared_f32(&sc[row], m);
      };
#if KVLR_ROUTE_ROLLING
      // Rolling prefetch: as soon as a 16-byte chunk of this row has been
      // consumed, the same chunk of the wave's next row is requested into the
      // freed registers, so about one row per wave stays in flight at no
      // extra register cost.
      int r = row0 + wave;
      uint4 vc[CV], kc[CK];
      if (r < row1) {
        const uint8_t *vb, *kb;
        const bool ok = row_base(r, vb, kb);
#pragma unroll
        for (int c = 0; c < CV; ++c) vc[c] = ok ? load16_stream(vb + c * kWave * 16) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int c = 0; c < CK; ++c) kc[c] = ok ? load16_stream(kb + c * kWave * 16) : make_uint4(0, 0, 0, 0);
      }
      for (; r < row1; r += kWaves) {
        const int rn = r + kWaves;
        const uint8_t *vbn = v_lat, *kbn = k_lat;
        const bool okn = (rn < row1) ? row_base(rn, vbn, kbn) : false;
        float acc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = 0.f;
        static_for<0, CV>([&](auto cc) {
          constexpr int C = decltype(cc)::value;
          float x[CH];
          S::unpack(vc[C], x);
          fma_heads_bcast<G, CH, W, C * CH>(qv, x, acc);
          vc[C] = okn ? load16_stream(vbn + C * kWave * 16) : make_uint4(0, 0, 0, 0);
        });
        static_for<0, CK>([&](auto cc) {
          constexpr int C = decltype(cc)::value;
          float x[CH];
          S::unpack(kc[C], x);
          fma_heads_bcast<G, CH, W, RV + C * CH>(qv, x, acc);
          kc[C] = okn ? load16_stream(kbn + C * kWave * 16) : make_uint4(0, 0, 0, 0);
        });
        finish_row(r, acc);
      }
#else
      for (int r = row0 + wave; r < row1; r += kWaves) {
        uint4 vc[CV], kc[CK];
        const uint8_t *vb, *kb;
        const bool ok = row_base(r, vb, kb);
#pragma unroll
        for (int c = 0; c < CV; ++c) vc[c] = ok ? load16_stream(vb + c * kWave * 16) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int c = 0; c < CK; ++c) kc[c] = ok ? load16_stream(kb + c * kWave * 16) : make_uint4(0, 0, 0, 0);
        float acc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = 0.f;
        static_for<0, CV>([&](auto cc) {
          constexpr int C = decltype(cc)::value;
          float x[CH];
          S::unpack(vc[C], x);
          fma_heads_bcast<G, CH, W, C * CH>(qv, x, acc);
        });
        static_for<0, CK>([&](auto cc) {
          constexpr int C = decltype(cc)::value;
          float x[CH];
          S::unpack(kc[C], x);
          fma_heads_bcast<G, CH, W, RV + C * CH>(qv, x, acc);
        });
        finish_row(r, acc);
      }
#endif
    } else {
      for (int row = row0 + wave; row < row1; row += kWaves) {
        const int t = row * kWave + lane;
        const bool valid = t < L;
        const int j = t >> log2P;
        const int slot = t & (P - 1);
        uint4 vc[CV], kc[CK];
        if (valid) {
          const size_t phys = static_cast<size_t>(pt[j]);
          const uint8_t* vbase = v_lat + (phys * Hkv + g) * slab_v + slot * 16;
          const uint8_t* kbase = k_lat + (phys * Hkv + g) * slab_k + slot * 16;
#pragma unroll
          for (int c = 0; c < CV; ++c) vc[c] = load16_stream(vbase + static_cast<size_t>(c) * P * 16);
#pragma unroll
          for (int c = 0; c < CK; ++c) kc[c] = load16_stream(kbase + static_cast<size_t>(c) * P * 16);
        } else {
#pragma unroll
          for (int c = 0; c < CV; ++c) vc[c] = make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int c = 0; c < CK; ++c) kc[c] = make_uint4(0, 0, 0, 0);
        }
        float m = row_score<S, G, RV, RK>(qv, vc, kc);
        if (!valid) m = -__builtin_huge_valf();
        m = row16_max(m);
        if (P == 32) m = fmaxf(m, __shfl_xor(m, 16, kWave));
        if (slot == 0 && valid) store_shared_f32(&sc[j], m);
      }
    }

    if (scores_only) {
      // page scores only (the selection runs where they are read): the
      // pair's first chunk marks the pages past the sequence
      if (split == 0)
        for (int j = ((L + P - 1) >> log2P) + static_cast<int>(threadIdx.x); j < max_pages; j += kThreads)
          sc[j] = -__builtin_huge_valf();
      continue;
    }
    // Ticket: the last chunk of this pair selects its pages.
    wait_stores_done();
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t prev = take_ticket(&counters[pair]);
      s_last = (prev == static_cast<uint32_t>(nsplit - 1));
    }
    __syncthreads();
    if (s_last) {
      const int N = (L + P - 1) >> log2P;
      // pages kept: the caller's per-sequence budget, else the fraction
      // (at least one page of a non-empty sequence); at most k_max
      const int k = pages_to_keep(N, k_pages, b, topk_num, topk_den, k_max);
      select_top_pages(sc, N, k, k_max, max_pages, sel + static_cast<size_t>(pair) * k_max, pt,
                       sel_phys ? sel_phys + static_cast<size_t>(pair) * k_max : nullptr);
      if (threadIdx.x == 0) {
        if (sel_counts) sel_counts[pair] = k;
        reset_ticket(&counters[pair]);
      }
    }
    __syncthreads();
  }
}

template <class S, int G, int RV, int RK>
hipError_t launch_t(const RouteArgs& a, hipStream_t s) {
  const int log2P = __builtin_ctz(static_cast<unsigned>(a.dm.P));
  const size_t lds = static_cast<size_t>(a.batch + 1) * sizeof(int);
  dim3 grid(a.grid);
  if (a.dm.P == kWave) {
    if (a.kl.adaptive) {
      if constexpr (S::CH == 8)  // per-head ranks: matrix-core path (bf16 or FP8 latents) only
        hipLaunchKernelGGL((route_kernel<S, G, RV, RK, true, true>), grid, dim3(kThreads), lds, s,
                           static_cast<const uint8_t*>(a.v_lat), static_cast<const uint8_t*>(a.k_lat),
                           a.q_proj, a.seq_lens, a.page_table, a.scores, a.counters, a.sel,
                           a.sel_counts, a.sel_phys, a.k_pages, a.dm.Hq, a.dm.Hkv, a.dm.P, log2P, a.max_pages, a.topk_num,
                           a.topk_den, a.k_max, a.rows_per_chunk, a.static_splits, a.scores_only, a.batch, a.kl);
      else
        return hipErrorInvalidValue;
    } else {
      hipLaunchKernelGGL((route_kernel<S, G, RV, RK, true>), grid, dim3(kThreads), lds, s,
                         static_cast<const uint8_t*>(a.v_lat), static_cast<const uint8_t*>(a.k_lat),
                         a.q_proj, a.seq_lens, a.page_table, a.scores, a.counters, a.sel, a.sel_counts,
                         a.sel_phys, a.k_pages, a.dm.Hq, a.dm.Hkv, a.dm.P, log2P, a.max_pages, a.topk_num, a.topk_den,
                         a.k_max, a.rows_per_chunk, a.static_splits, a.scores_only, a.batch, a.kl);
    }
  } else {
    if constexpr (S::CB == 8) return hipErrorInvalidValue;  // FP8 latents: 64-token pages only
    else
      hipLaunchKernelGGL((route_kernel<S, G, RV, RK, false>), grid, dim3(kThreads), lds, s,
                         static_cast<const uint8_t*>(a.v_lat), static_cast<const uint8_t*>(a.k_lat),
                         a.q_proj, a.seq_lens, a.page_table, a.scores, a.counters, a.sel, a.sel_counts,
                         a.sel_phys, a.k_pages, a.dm.Hq, a.dm.Hkv, a.dm.P, log2P, a.max_pages, a.topk_num, a.topk_den,
                         a.k_max, a.rows_per_chunk, a.static_splits, a.scores_only, a.batch, a.kl);
  }
  return hipGetLastError();
}

template <class S, int G, int RV>
hipError_t by_rk(const RouteArgs& a, hipStream_t s) {
  switch (a.dm.RK) {
    case 16: return launch_t<S, G, RV, 16>(a, s);
    case 32: return launch_t<S, G, RV, 32>(a, s);
    case 64: return launch_t<S, G, RV, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class S, int G>
hipError_t by_rv(const RouteArgs& a, hipStream_t s) {
  switch (a.dm.RV) {
    case 16: return by_rk<S, G, 16>(a, s);
    case 32: return by_rk<S, G, 32>(a, s);
    case 64: return by_rk<S, G, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class S>
hipError_t by_g(const RouteArgs& a, hipStream_t s) {
  switch (a.dm.G) {
    case 1: return by_rv<S, 1>(a, s);
    case 2: return by_rv<S, 2>(a, s);
    case 4: return by_rv<S, 4>(a, s);
    case 8: return by_rv<S, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

#ifndef KVLR_ROUTE_RPC
#define KVLR_ROUTE_RPC 64
#endif
// Rows of at most 8 KB (rank_v + rank_k <= 64 with bf16 latents, <= 128 with
// FP8) can take a chunk size of their own. With the selection in a launch of
// its own a chunk's fixed costs are small, and 64 rows measured best for
// every row size (128 kept only while each chunk ended with a ticket).
#ifndef KVLR_ROUTE_RPC_SMALL
#define KVLR_ROUTE_RPC_SMALL KVLR_ROUTE_RPC  // rows of at most 8 KB
#endif
int route_rows_per_chunk(int row_bytes) { return row_bytes <= 8192 ? KVLR_ROUTE_RPC_SMALL : KVLR_ROUTE_RPC; }

#ifndef KVLR_ROUTE_TICKET
#define KVLR_ROUTE_TICKET 0  // 1: select in the routing launch (last workgroup of each pair, a ticket)
#endif

// Routing: the scoring launch, then (unless scores only) the selection
// launch; with KVLR_ROUTE_TICKET the selection runs inside the scoring launch.
hipError_t launch_route(const RouteArgs& a0, hipStream_t s) {
  if (a0.batch == 0) return hipSuccess;
  RouteArgs a = a0;
  const bool separate = !a.scores_only && !KVLR_ROUTE_TICKET;
  if (separate) a.scores_only = 1;
  hipError_t e;
  if (a.dm.lat == 2) e = by_g<FP8>(a, s);
  else if (a.dm.lat == 0) e = by_g<BF16>(a, s);
  else e = by_g<F32>(a, s);
  if (e != hipSuccess || !separate) return e;
  return launch_select(a, s);
}

#ifndef KVLR_SELECT_512
#define KVLR_SELECT_512 1  // 512-thread selection workgroups for tables of 257 .. 1024 pages
#endif
hipError_t launch_select(const RouteArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const int log2P = __builtin_ctz(static_cast<unsigned>(a.dm.P));
  if (a.max_pages > 1024 && a.max_pages <= kSelectLds)
    hipLaunchKernelGGL(select_kernel<1024>, dim3(a.batch * a.dm.Hkv), dim3(1024), 0, s, a.scores,
                       a.seq_lens, a.page_table, a.sel, a.sel_counts, a.sel_phys, a.k_pages, a.dm.Hkv,
                       a.dm.P, log2P, a.max_pages, a.topk_num, a.topk_den, a.k_max);
  else if (KVLR_SELECT_512 && a.max_pages > 256 && a.max_pages <= 1024)
    hipLaunchKernelGGL(select_kernel<512>, dim3(a.batch * a.dm.Hkv), dim3(512), 0, s, a.scores,
                       a.seq_lens, a.page_table, a.sel, a.sel_counts, a.sel_phys, a.k_pages, a.dm.Hkv,
                       a.dm.P, log2P, a.max_pages, a.topk_num, a.topk_den, a.k_max);
  else
    hipLaunchKernelGGL(select_kernel<kThreads>, dim3(a.batch * a.dm.Hkv), dim3(kThreads), 0, s,
                       a.scores, a.seq_lens, a.page_table, a.sel, a.sel_counts, a.sel_phys, a.k_pages,
                       a.dm.Hkv, a.dm.P, log2P, a.max_pages, a.topk_num, a.topk_den, a.k_max);
  return hipGetLastError();
}

}  // namespace kvlr
