// Decode attention over the compressed cache, value side in latent space.
//
// BasisKV: Value Latents for Communication and Key Routing, English abstract:
// the original keys are read only for the selected pages and give exact QK
// scores; the value cache holds rank-r_v latents and value compression is
// tied to the output projection, so the softmax-weighted sum stays in latent
// space, z = sum_t p_t v_t, and B_v is applied once per head afterwards.
// In the dense low-rank mode the keys are latents too: s_t = scale q B_k^T . k_t.
//
// Work split: a persistent grid walks a device-built list of chunks; a chunk
// is a run of up to rows_per_chunk 64-token rows of one (sequence, KV head)
// pair's page list (selected pages, or all pages), and the 4 waves of a
// workgroup take every fourth row of it. Per row:
//   scores  - one lane per token; the token's key row is read as 16-byte
//             chunks (contiguous across the row's tokens), the wave-uniform
//             query is read with scalar loads; G heads share each load;
//   softmax - online (running max and sum per head, base-2 exponent);
//   P.V     - lanes regroup as (latent chunk c, tokens l/CV + k*64/CV), the
//             probabilities are exchanged through LDS, each lane accumulates
//             G x CH latent outputs.
// With one page per row (page_size 64) every key and value register is
// re-requested with the wave's next row as soon as it has been used, so each
// wave keeps a row in flight.
// The waves of a workgroup merge their (max, sum, z) partials in LDS and the
// workgroup writes one partial record per chunk; merge_kernel (a second
// launch) combines a pair's chunk records into z and lse, and with B_v given
// applies the up-projection o_h = z_h B_v there, once per query head.
//
// Chunk plan: with page ids and no per-pair counts, every pair walks k_max
// rows (ids of -1 are skipped), so a chunk's pair and split follow from its
// index alone and nothing is read before the chunk's own page ids; with
// counts (ragged batches) or without page ids (every page), each workgroup
// first builds the per-sequence prefix of chunk counts in LDS.

#include "kvlr_device.h"
#include "kvlr_internal.h"

#ifndef KVLR_ATTN_MFMA
#define KVLR_ATTN_MFMA 1
#endif
#ifndef KVLR_ATTN_ROWS_SELECTED
#define KVLR_ATTN_ROWS_SELECTED 16
#endif
#ifndef KVLR_ATTN_ROWS_DENSE
#define KVLR_ATTN_ROWS_DENSE 128
#endif

namespace kvlr {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ inline void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Chunks of one pair when chunk counts come from the per-sequence plan: the
// most items (pages) over the sequence's KV heads, in rows of 64 tokens,
// split into runs of rows_per_chunk rows (at least one chunk).
template <class ItemsFn>
__device__ inline int attn_splits(ItemsFn items_of, int b, int Hkv, int ipr_log2, int rpc) {
  int items = 0;
  for (int g = 0; g < Hkv; ++g) items = max(items, items_of(b, g));
  const int rows = (items + (1 << ipr_log2) - 1) >> ipr_log2;
  return max(1, (rows + rpc - 1) / rpc);
}

// S: storage of the keys the scores read (original keys, or key latents);
// SV: storage of the value latents. With FP8 latents S is BF16 (original
// keys) or FP8 (key latents), SV is FP8, and the factors are bf16.
template <class S, class SV, int G, int KW, int RV, bool ROWPAGE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_kernel(
    const uint8_t* __restrict__ keys, const uint8_t* __restrict__ v_lat,
    const float* __restrict__ qsrc, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ sel_phys, const int32_t* __restrict__ sel_counts,
    float* __restrict__ partials, int Hq, int Hkv, int P, int log2P, int max_pages, int k_max,
    float scale_log2e, int rows_per_chunk, int max_splits, int batch) {
  constexpr int CH = S::CH;
  static_assert(SV::CH == CH, "keys and value latents share the elements per chunk");
  constexpr int CKW = KW / CH;     // key chunks per token
  constexpr int CV = RV / CH;      // value-latent chunks per token
  constexpr int TPL = kWave / CV;  // token stride between a lane's P.V tokens
  constexpr int PW = RV + 2;       // partial record: m, l, z[RV]

  extern __shared__ int s_base[];
  __shared__ float s_p[kWaves][kWave][G];
  __shared__ float s_ml[kWaves][G][2];
  __shared__ float s_z[kWaves][G][RV];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int ipr_log2 = 6 - log2P;  // items (pages) per row = 64 / P
  const size_t slab_k = static_cast<size_t>(CKW) * P * S::CB;
  const size_t slab_v = static_cast<size_t>(CV) * P * SV::CB;
  const int my_c = lane % CV;

  // attended items (pages) of a (sequence, KV head) pair
  auto items_of = [&](int b, int g) {
    if (!sel) return (table_len(seq_lens[b], max_pages, P) + P - 1) >> log2P;
    return sel_counts ? min(max(sel_counts[b * Hkv + g], 0), k_max) : k_max;
  };
  const bool uniform = sel && !sel_counts;  // every pair walks k_max rows in max_splits chunks
  int total;
  if (uniform) {
    total = batch * Hkv * max_splits;
  } else {
    build_chunk_prefix(batch, s_base,
                       [&](int b) { return Hkv * attn_splits(items_of, b, Hkv, ipr_log2, rows_per_chunk); });
    total = s_base[batch];
  }

  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    int b, g, split, nsplit;
    if (uniform) {
      const int pr = w / max_splits;
      split = w - pr * max_splits;
      nsplit = max_splits;
      b = pr / Hkv;
      g = pr - b * Hkv;
    } else {
      b = find_sequence(s_base, batch, w);
      nsplit = (s_base[b + 1] - s_base[b]) / Hkv;
      const int local = w - s_base[b];
      g = local / nsplit;
      split = local - g * nsplit;
    }
    const int L = table_len(seq_lens[b], max_pages, P);
    const int N = (L + P - 1) >> log2P;
    const int n_items = items_of(b, g);
    const int nrows = (n_items + (1 << ipr_log2) - 1) >> ipr_log2;
    const int pair = b * Hkv + g;
    const int32_t* __restrict__ pt = page_table + static_cast<size_t>(b) * max_pages;
    const int32_t* __restrict__ sl = sel ? sel + static_cast<size_t>(pair) * k_max : nullptr;
    // physical pages of the selected ids (written by routing beside them), or
    // the page table
    const int32_t* __restrict__ sp = (sel && sel_phys) ? sel_phys + static_cast<size_t>(pair) * k_max : nullptr;
    auto phys_of = [&](int row, int pg) -> size_t {
      return static_cast<size_t>(sp ? sp[row] : pt[pg]);
    };
    const float* __restrict__ qg = qsrc + static_cast<size_t>(b * Hq + g * G) * KW;
    const int row0 = split * rows_per_chunk;
    const int row1 = min(row0 + rows_per_chunk, nrows);
    // (FP8 latents have only the matrix-core path)
    constexpr bool kMfma = ROWPAGE && S::CH == 8 && (KVLR_ATTN_MFMA || SV::CB == 8);

    float m[G], lsum[G], z[G][CH];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kNegInf;
      lsum[h] = 0.f;
#pragma unroll
      for (int e = 0; e < CH; ++e) z[h][e] = 0.f;
    }

    // online softmax update for one row's scores; returns false if nothing valid yet
    auto softmax_row = [&](float (&s)[G], bool valid) -> bool {
      bool any = false;
      float p[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float sv = valid ? s[h] * scale_log2e : kNegInf;
        const float mx = wave_max_u(sv);
        const float mn = fmaxf(m[h], mx);
        any = any || (mn != kNegInf);
        const float alpha = (mn == kNegInf) ? 1.f : fast_exp2(m[h] - mn);
        p[h] = (mn == kNegInf) ? 0.f : fast_exp2(sv - mn);
        lsum[h] = lsum[h] * alpha + p[h];
#pragma unroll
        for (int e = 0; e < CH; ++e) z[h][e] *= alpha;
        m[h] = mn;
      }
      if (any) {
#pragma unroll
        for (int h = 0; h < G; ++h) s_p[wave][lane][h] = p[h];
        wave_lds_sync();
      }
      return any;
    };
    auto accumulate_pv = [&](const typename SV::Raw (&vc)[CV]) {
#pragma unroll
      for (int k = 0; k < CV; ++k) {
        const int tok = lane / CV + k * TPL;
        float x[CH];
        SV::unpack(vc[k], x);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pp = s_p[wave][tok][h];
#pragma unroll
          for (int e = 0; e < CH; ++e) z[h][e] = fmaf(pp, x[e], z[h][e]);
        }
      }
      wave_lds_sync();
    };
    auto score_keys = [&](const typename S::Raw (&kc)[CKW], float (&s)[G]) {
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = 0.f;
      static_for<0, CKW>([&](auto cc) {
        constexpr int C = decltype(cc)::value;
        float x[CH];
        S::unpack(kc[C], x);
        fma_heads<G, CH, KW, C * CH>(qg, x, s);
      });
    };

    if constexpr (kMfma) {
      // Matrix-core scores (bf16 storage, one page per row): a 64-token row is
      // four 16-token tiles, scores[token][head] from v_mfma_f32_16x16x32_bf16
      // with tokens as rows (lane l: token l%16, one 16-byte key chunk from
      // k-group l/16) and heads as columns (the queries split into bf16 high
      // and low halves, two products per step; exact to about 2^-18 relative).
      // Lane l then holds head l%16's scores of tokens 16j + 4(l/16) + v. The
      // row max per head comes from two cross-lane steps; the running max and
      // rescale stay wave-uniform per head, each lane keeps a partial sum of
      // its own probabilities, and P.V runs as in the vector path.
      constexpr int KS = (CKW + 3) / 4;  // k-steps of 32 key elements
      const int kq = lane >> 4, col = lane & 15;
      // the query halves, one 16-byte fragment per (k-step, half, lane), live
      // in the wave's LDS slice and are read once per k-step of a row. The
      // query is requested first, the first rows' page ids next and their
      // key and value chunks after those arrive; the halves are formed and
      // stored only then, so the chunk's start waits for two memory round
      // trips (query with page ids, then the first rows) instead of three.
      __shared__ uint4 s_qf[kWaves][KS][2][kWave];
      float4 qx[KS][2];
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const int ci = 4 * st + kq;
        if (col < G && ci < CKW) {
          const float* src = qg + col * KW + ci * 8;
          qx[st][0] = *reinterpret_cast<const float4*>(src);
          qx[st][1] = *reinterpret_cast<const float4*>(src + 4);
        } else {
          qx[st][0] = qx[st][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      auto stage_query = [&] {
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          const float x[8] = {qx[st][0].x, qx[st][0].y, qx[st][0].z, qx[st][0].w,
                              qx[st][1].x, qx[st][1].y, qx[st][1].z, qx[st][1].w};
          bf16x8 hi, lo;
          split_bf16x8(x, hi, lo);
          s_qf[wave][st][0][lane] = __builtin_bit_cast(uint4, hi);
          s_qf[wave][st][1][lane] = __builtin_bit_cast(uint4, lo);
        }
        wave_lds_sync();
      };
      // With chosen page ids and at most 64 rows per chunk, lane l reads the
      // id (and physical page) of the chunk's row l, one request per array
      // issued with the query's; every row's lookup, the first ones and the
      // loop's (two and three rows ahead), is then a read of a lane with no
      // memory round trip of its own. Otherwise each lookup reads memory.
      const bool lanes = sl != nullptr && rows_per_chunk <= kWave;
      int lane_pg = -1, lane_ph = 0;
      if (lanes) {
        const int li = row0 + lane < row1 ? row0 + lane : 0;
        lane_pg = sl[li];
        if (sp) lane_ph = sp[li];
      }
      auto page_of = [&](int row) -> int {
        if (row >= row1) return -1;
        const int pg = lanes ? __builtin_amdgcn_readlane(lane_pg, row - row0) : (sl ? sl[row] : row);
        return (pg >= 0 && pg < N) ? pg : -1;
      };
      // past the last row every lane reads one shared address (on = 0);
      // past the last key chunk a lane re-reads chunk 0 (its query half is zero)
      struct RowRef {
        const uint8_t* kb;
        const uint8_t* vb;
        int on, nvalid;
      };
      auto row_ref = [&](int row, int pg) -> RowRef {
        if (pg < 0) return RowRef{keys, v_lat, 0, 0};
        const size_t ph = (lanes && sp) ? static_cast<size_t>(__builtin_amdgcn_readlane(lane_ph, row - row0))
                                        : phys_of(row, pg);
        return RowRef{keys + (ph * Hkv + g) * slab_k,
                      v_lat + (ph * Hkv + g) * slab_v + my_c * kWave * SV::CB, 1,
                      min(L - pg * kWave, kWave)};
      };
      auto a_addr = [&](const RowRef& rr, int j, int st) -> const uint8_t* {
        int ci = 4 * st + kq;
        if (ci >= CKW) ci = 0;
        return rr.kb + static_cast<uint32_t>(rr.on) *
                           static_cast<uint32_t>((j * 16 + col) * S::CB + ci * (kWave * S::CB));
      };
      auto v_addr = [&](const RowRef& rr, int k) -> const uint8_t* {
        return rr.vb + static_cast<uint32_t>(rr.on) * static_cast<uint32_t>((lane / CV + k * TPL) * SV::CB);
      };
      int r = row0 + wave;
      typename S::Raw A[4][KS];
      typename SV::Raw vc[CV];
      RowRef cur = row_ref(r, page_of(r));
      RowRef nxt = row_ref(r + kWaves, page_of(r + kWaves));
      int pg2 = page_of(r + 2 * kWaves);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int st = 0; st < KS; ++st) A[j][st] = S::load_stream(a_addr(cur, j, st));
#pragma unroll
      for (int k = 0; k < CV; ++k) vc[k] = SV::load_stream(v_addr(cur, k));
      stage_query();
      float lcol = 0.f;  // sum of this lane's probabilities of head col
      for (; r < row1; r += kWaves) {
        // table lookups run ahead: physical page two rows on, page id three rows on
        const RowRef nn = row_ref(r + 2 * kWaves, pg2);
        const int pg3 = page_of(r + 3 * kWaves);
        f32x4 acc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          const bf16x8 qhi = __builtin_bit_cast(bf16x8, s_qf[wave][st][0][lane]);
          const bf16x8 qlo = __builtin_bit_cast(bf16x8, s_qf[wave][st][1][lane]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x8 a = S::to_bf16x8(A[j][st]);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qhi, acc[j], 0, 0, 0);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qlo, acc[j], 0, 0, 0);
            A[j][st] = S::load_stream(a_addr(nxt, j, st));
          }
        }
        // scaled score of (token 16j + 4kq + v, head col), -inf when masked
        auto score = [&](int j, int v) -> float {
          const bool ok = col < G && (j * 16 + 4 * kq + v) < cur.nvalid;
          return ok ? acc[j][v] * scale_log2e : kNegInf;
        };
        float rm = kNegInf;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) rm = fmaxf(rm, score(j, v));
        rm = fmaxf(rm, __shfl_xor(rm, 16, kWave));
        rm = fmaxf(rm, __shfl_xor(rm, 32, kWave));
        bool any = false;
        float mcol = kNegInf, acol = 1.f;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rm), h));
          const float mn = fmaxf(m[h], mx);
          const float alpha = (mn == kNegInf) ? 1.f : fast_exp2(m[h] - mn);
          any = any || (mn != kNegInf);
          m[h] = mn;
#pragma unroll
          for (int e = 0; e < CH; ++e) z[h][e] *= alpha;
          if (col == h) {
            mcol = mn;
            acol = alpha;
          }
        }
        lcol *= acol;
        if (any) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float sc = score(j, v);
              const float pv = (sc == kNegInf) ? 0.f : fast_exp2(sc - mcol);
              lcol += pv;
              if (col < G) s_p[wave][j * 16 + 4 * kq + v][col] = pv;
            }
          wave_lds_sync();
        }
#pragma unroll
        for (int k = 0; k < CV; ++k) {
          const int tok = lane / CV + k * TPL;
          if (any) {
            float x[CH];
            SV::unpack(vc[k], x);
            const bool tv = tok < cur.nvalid;
#pragma unroll
            for (int h = 0; h < G; ++h) {
              const float pp = s_p[wave][tok][h];
#pragma unroll
              for (int e = 0; e < CH; ++e) z[h][e] = fmaf(pp, tv ? x[e] : 0.f, z[h][e]);
            }
          }
          vc[k] = SV::load_stream(v_addr(nxt, k));
        }
        if (any) wave_lds_sync();
        cur = nxt;
        nxt = nn;
        pg2 = pg3;
      }
      // per-head probability sums: lanes col, col+16, col+32, col+48 hold
      // disjoint tokens; lane 0 carries each total into the reduction below
      lcol += __shfl_xor(lcol, 16, kWave);
      lcol += __shfl_xor(lcol, 32, kWave);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float t = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lcol), h));
        lsum[h] = (lane == 0) ? t : 0.f;
      }
    } else if constexpr (ROWPAGE) {
      // One page per row: page id and physical page are wave-uniform. Each
      // key or value register is re-requested with the next row's data as
      // soon as this row has used it, so a wave always has a row in flight.
      // The loads carry no branch (the compiler can then count them in
      // flight): past the last row every lane reads one shared address, and
      // slots past the sequence end are read but never used (scores are
      // masked, value chunks are zeroed when used).
      auto page_of = [&](int row) -> int {
        if (row >= row1) return -1;
        const int pg = sl ? sl[row] : row;
        return (pg >= 0 && pg < N) ? pg : -1;
      };
      struct RowRef {
        const uint8_t* kb;
        const uint8_t* vb;
        int kstride, vstride, nvalid;
      };
      auto row_ref = [&](int row, int pg) -> RowRef {
        RowRef rr;
        if (pg >= 0) {
          const size_t ph = phys_of(row, pg);
          rr.kb = keys + (ph * Hkv + g) * slab_k + lane * 16;
          rr.vb = v_lat + (ph * Hkv + g) * slab_v + my_c * kWave * 16;
          rr.kstride = kWave * 16;
          rr.vstride = 16;
          rr.nvalid = min(L - pg * kWave, kWave);
        } else {
          rr.kb = keys;
          rr.vb = v_lat;
          rr.kstride = 0;
          rr.vstride = 0;
          rr.nvalid = 0;
        }
        return rr;
      };
      int r = row0 + wave;
      uint4 kc[CKW], vc[CV];
      RowRef cur = row_ref(r, page_of(r));
#pragma unroll
      for (int c = 0; c < CKW; ++c) kc[c] = load16_stream(cur.kb + c * cur.kstride);
#pragma unroll
      for (int k = 0; k < CV; ++k) vc[k] = load16_stream(cur.vb + (lane / CV + k * TPL) * cur.vstride);
      RowRef nxt = row_ref(r + kWaves, page_of(r + kWaves));
      int pg2 = page_of(r + 2 * kWaves);
      for (; r < row1; r += kWaves) {
        // table lookups run ahead: physical page two rows on, page id three rows on
        const RowRef nn = row_ref(r + 2 * kWaves, pg2);
        const int pg3 = page_of(r + 3 * kWaves);
        float s[G];
#pragma unroll
        for (int h = 0; h < G; ++h) s[h] = 0.f;
        static_for<0, CKW>([&](auto cc) {
          constexpr int C = decltype(cc)::value;
          float x[CH];
          S::unpack(kc[C], x);
          fma_heads<G, CH, KW, C * CH>(qg, x, s);
          kc[C] = load16_stream(nxt.kb + C * nxt.kstride);
        });
        const bool use = (cur.nvalid > 0) && softmax_row(s, lane < cur.nvalid);
#pragma unroll
        for (int k = 0; k < CV; ++k) {
          const int tok = lane / CV + k * TPL;
          if (use) {
            float x[CH];
            S::unpack(vc[k], x);
            const bool tv = tok < cur.nvalid;
#pragma unroll
            for (int h = 0; h < G; ++h) {
              const float pp = s_p[wave][tok][h];
#pragma unroll
              for (int e = 0; e < CH; ++e) z[h][e] = fmaf(pp, tv ? x[e] : 0.f, z[h][e]);
            }
          }
          vc[k] = load16_stream(nxt.vb + tok * nxt.vstride);
        }
        if (use) wave_lds_sync();
        cur = nxt;
        nxt = nn;
        pg2 = pg3;
      }
    } else {
      for (int row = row0 + wave; row < row1; row += kWaves) {
        const int item = (row << ipr_log2) + (lane >> log2P);
        const int slot = lane & (P - 1);
        int page = -1;
        if (item < n_items) page = sl ? sl[item] : item;
        const bool valid = page >= 0 && page < N && (page << log2P) + slot < L;
        const int phys = valid ? static_cast<int>(phys_of(item, page)) : 0;
        uint4 kc[CKW];
        if (valid) {
          const uint8_t* kb = keys + (static_cast<size_t>(phys) * Hkv + g) * slab_k + slot * 16;
#pragma unroll
          for (int c = 0; c < CKW; ++c) kc[c] = load16_stream(kb + static_cast<size_t>(c) * P * 16);
        } else {
#pragma unroll
          for (int c = 0; c < CKW; ++c) kc[c] = make_uint4(0, 0, 0, 0);
        }
        uint4 vc[CV];
#pragma unroll
        for (int k = 0; k < CV; ++k) {
          const int tok = lane / CV + k * TPL;
          const int tphys = __shfl(phys, tok, kWave);
          const int tvalid = __shfl(static_cast<int>(valid), tok, kWave);
          vc[k] = make_uint4(0, 0, 0, 0);
          if (tvalid) {
            const int tslot = tok & (P - 1);
            vc[k] = load16_stream(v_lat + (static_cast<size_t>(tphys) * Hkv + g) * slab_v +
                                  static_cast<size_t>(my_c) * P * 16 + tslot * 16);
          }
        }
        float s[G];
        score_keys(kc, s);
        if (softmax_row(s, valid)) accumulate_pv(vc);
      }
    }

    // ---- wave reduction: lanes with the same chunk hold disjoint token sets
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int off = CV; off < kWave; off <<= 1)
#pragma unroll
        for (int e = 0; e < CH; ++e) z[h][e] += __shfl_xor(z[h][e], off, kWave);
      lsum[h] = wave_sum_u(lsum[h]);
    }
    if (lane < CV) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < CH; ++e) s_z[wave][h][lane * CH + e] = z[h][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s_ml[wave][h][0] = m[h];
        s_ml[wave][h][1] = lsum[h];
      }
    }
    __syncthreads();

    // ---- chunk partial (max, sum, z) per head; merge_kernel combines them
    float* part = partials + (static_cast<size_t>(pair) * max_splits + split) * G * PW;
    for (int i = threadIdx.x; i < G * RV; i += kThreads) {
      const int h = i / RV, e = i - h * RV;
      float M = kNegInf;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, s_ml[ww][h][0]);
      float Z = 0.f, Ls = 0.f;
      if (M != kNegInf) {
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
          const float f = fast_exp2(s_ml[ww][h][0] - M);
          Z += f * s_z[ww][h][e];
          Ls += f * s_ml[ww][h][1];
        }
      }
      part[h * PW + 2 + e] = Z;
      if (e == 0) {
        part[h * PW] = M;
        part[h * PW + 1] = Ls;
      }
    }
    __syncthreads();
  }
}

// Combines the chunk records of each (sequence, KV head) pair: with M the
// largest chunk max (base-2 scaled scores), z = sum_c 2^(m_c - M) z_c /
// sum_c 2^(m_c - M) l_c and lse = (M + log2 l) ln 2; no valid token gives
// z = 0, lse = -inf. With B_v, o_h = z_h B_v[g] for the group's heads.
// One workgroup per pair; the pair's chunk count follows the attention
// launch's plan. Every load of a chunk record is issued before the first is
// used; B_v is staged in LDS meanwhile.
template <class SF, int G, int RV>
__global__ __launch_bounds__(kThreads) void merge_kernel(
    const float* __restrict__ partials, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_counts, int k_max,
    int P, int log2P, int max_pages, int rows_per_chunk, int max_splits, int Hq, int Hkv, int Dh,
    float* __restrict__ z_out, float* __restrict__ lse_out, const uint8_t* __restrict__ B_v,
    float* __restrict__ o_out) {
  constexpr int PW = RV + 2;
  __shared__ float s_zz[G][RV];
  __shared__ uint4 s_bv[RV * 128 * SF::ELEM_BYTES / 16];  // B_v[g] as stored, head_dim <= 128
  const int pair = blockIdx.x;
  const int b = pair / Hkv, g = pair - b * Hkv;
  const int ipr_log2 = 6 - log2P;
  auto items_of = [&](int bb, int gg) {
    if (!sel) return (table_len(seq_lens[bb], max_pages, P) + P - 1) >> log2P;
    return sel_counts ? min(max(sel_counts[bb * Hkv + gg], 0), k_max) : k_max;
  };
  const int nsplit = (sel && !sel_counts) ? max_splits
                                          : attn_splits(items_of, b, Hkv, ipr_log2, rows_per_chunk);
  // B_v[g] is requested together with the records (one round trip for
  // both) and written to LDS once the records are merged
  constexpr int NBV = (RV * 128 * SF::ELEM_BYTES / 16 + kThreads - 1) / kThreads;
  const int nbv = RV * Dh * SF::ELEM_BYTES / 16;
  uint4 bv[NBV];
  if (o_out) {
    const uint8_t* Bg = B_v + static_cast<size_t>(g) * RV * Dh * SF::ELEM_BYTES;
#pragma unroll
    for (int it = 0; it < NBV; ++it) {
      const int i = static_cast<int>(threadIdx.x) + it * kThreads;
      bv[it] = load16(Bg + static_cast<size_t>(i < nbv ? i : 0) * 16);
    }
  }
  const float* allp = partials + static_cast<size_t>(pair) * max_splits * G * PW;
  for (int i = threadIdx.x; i < G * RV; i += kThreads) {
    const int h = i / RV, e = i - h * RV;
    float M = kNegInf, Z = 0.f, Ls = 0.f;
    for (int sp0 = 0; sp0 < nsplit; sp0 += 8) {
      float mm[8], ll[8], zz[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {  // past the last chunk: re-read it, skipped below
        const float* r = allp + (min(sp0 + u, nsplit - 1) * G + h) * PW;
        mm[u] = r[0];
        ll[u] = r[1];
        zz[u] = r[2 + e];
      }
      // (selects, not a branch: the loads of every record are then used
      // unconditionally and go out together)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool ok = sp0 + u < nsplit && mm[u] != kNegInf;
        const float mn = ok ? fmaxf(M, mm[u]) : M;
        const float a = (M == kNegInf) ? 0.f : fast_exp2(M - mn);
        const float f = fast_exp2(mm[u] - mn);
        const float zn = Z * a + f * zz[u];
        const float ln = Ls * a + f * ll[u];
        Z = ok ? zn : Z;
        Ls = ok ? ln : Ls;
        M = mn;
      }
    }
    const int qh = g * G + h;
    const float zv = (Ls > 0.f) ? Z / Ls : 0.f;
    z_out[(static_cast<size_t>(b) * Hq + qh) * RV + e] = zv;
    s_zz[h][e] = zv;
    if (e == 0 && lse_out)
      lse_out[static_cast<size_t>(b) * Hq + qh] =
          (Ls > 0.f) ? (M + fast_log2(Ls)) * 0.69314718055994530942f : kNegInf;
  }
  if (o_out) {
    // value compression tied to the output projection: o_h = z_h B_v, once
    // per head. A thread takes 4 consecutive outputs of one head over a
    // contiguous 1/ES of the latent index; the ES partial sums sit in
    // adjacent lanes and are added with two-lane exchanges.
#pragma unroll
    for (int it = 0; it < NBV; ++it) {
      const int i = static_cast<int>(threadIdx.x) + it * kThreads;
      if (i < nbv) s_bv[i] = bv[it];
    }
    __syncthreads();
    const int nq = Dh >> 2;                 // 4-output groups per head
    int es = kThreads / (G * nq);           // latent splits per group: 1 .. 8
    es = es >= 8 ? 8 : es >= 4 ? 4 : es >= 2 ? 2 : 1;
    const int item = threadIdx.x / es, part = threadIdx.x - item * es;
    const bool on = item < G * nq;
    const int h = on ? item / nq : 0, d0 = on ? (item - (item / nq) * nq) * 4 : 0;
    const int e0 = part * (RV / es), e1 = e0 + RV / es;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int e = e0; e < e1; ++e) {
      const float zv = s_zz[h][e];
      float bv[4];
      SF::load4(s_bv, static_cast<long>(e) * Dh + d0, bv);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fmaf(zv, bv[j], acc[j]);
    }
    for (int m = 1; m < es; m <<= 1)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += __shfl_xor(acc[j], m);
    if (on && part == 0)
      *reinterpret_cast<float4*>(o_out + (static_cast<size_t>(b) * Hq + g * G + h) * Dh + d0) =
          make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
}

template <class S, class SV, int G, int KW, int RV>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  if (a.q_stride != KW) return hipErrorInvalidValue;  // queries are read with stride KW
  const int log2P = __builtin_ctz(static_cast<unsigned>(a.dm.P));
  const size_t lds = static_cast<size_t>(a.batch + 1) * sizeof(int);
  dim3 grid(a.grid);
  if constexpr (SV::CB == 8) {  // FP8 latents: 64-token pages only
    if (a.dm.P != kWave) return hipErrorInvalidValue;
  }
  if (a.dm.P == kWave)
    hipLaunchKernelGGL((attn_kernel<S, SV, G, KW, RV, true>), grid, dim3(kThreads), lds, s,
                       static_cast<const uint8_t*>(a.keys), static_cast<const uint8_t*>(a.v_lat),
                       a.qsrc, a.seq_lens, a.page_table, a.sel, a.sel_phys, a.sel_counts,
                       a.partials, a.dm.Hq, a.dm.Hkv, a.dm.P, log2P, a.max_pages, a.k_max,
                       a.scale_log2e, a.rows_per_chunk, a.max_splits, a.batch);
  else if constexpr (SV::CB == 16)
    hipLaunchKernelGGL((attn_kernel<S, SV, G, KW, RV, false>), grid, dim3(kThreads), lds, s,
                       static_cast<const uint8_t*>(a.keys), static_cast<const uint8_t*>(a.v_lat),
                       a.qsrc, a.seq_lens, a.page_table, a.sel, a.sel_phys, a.sel_counts,
                       a.partials, a.dm.Hq, a.dm.Hkv, a.dm.P, log2P, a.max_pages, a.k_max,
                       a.scale_log2e, a.rows_per_chunk, a.max_splits, a.batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  using SF = std::conditional_t<S::CB == 8, BF16, S>;  // factor storage
  hipLaunchKernelGGL((merge_kernel<SF, G, RV>), dim3(a.batch * a.dm.Hkv), dim3(kThreads), 0, s,
                     a.partials, a.seq_lens, a.sel, a.sel_counts, a.k_max, a.dm.P, log2P, a.max_pages,
                     a.rows_per_chunk, a.max_splits, a.dm.Hq, a.dm.Hkv, a.dm.D, a.z_out, a.lse_out,
                     static_cast<const uint8_t*>(a.B_v), a.o_out);
  return hipGetLastError();
}

template <class S, class SV, int G, int RV>
hipError_t by_kw(const AttnArgs& a, hipStream_t s) {
  // key width: head_dim for original keys, rank_k for key latents
  switch (a.dm.exact ? a.dm.D : a.dm.RK) {
    case 16: return launch_t<S, SV, G, 16, RV>(a, s);
    case 32: return launch_t<S, SV, G, 32, RV>(a, s);
    case 64: return launch_t<S, SV, G, 64, RV>(a, s);
    case 128: return launch_t<S, SV, G, 128, RV>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class S, class SV, int G>
hipError_t by_rv(const AttnArgs& a, hipStream_t s) {
  switch (a.dm.RV) {
    case 16: return by_kw<S, SV, G, 16>(a, s);
    case 32: return by_kw<S, SV, G, 32>(a, s);
    case 64: return by_kw<S, SV, G, 64>(a, s);
    case 128:  // values at full width: bf16 only
      if constexpr (std::is_same_v<S, BF16> && std::is_same_v<SV, BF16>) return by_kw<S, SV, G, 128>(a, s);
      break;
  }
  return hipErrorInvalidValue;
}

template <class S, class SV>
hipError_t by_g(const AttnArgs& a, hipStream_t s) {
  switch (a.dm.G) {
    case 1: return by_rv<S, SV, 1>(a, s);
    case 2: return by_rv<S, SV, 2>(a, s);
    case 4: return by_rv<S, SV, 4>(a, s);
    case 8: return by_rv<S, SV, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int attn_rows_per_chunk(bool selected) {
  return selected ? KVLR_ATTN_ROWS_SELECTED : KVLR_ATTN_ROWS_DENSE;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  if (a.dm.lat == 2) return a.dm.exact ? by_g<BF16, FP8>(a, s) : by_g<FP8, FP8>(a, s);
  if (a.dm.dtype == 0) return by_g<BF16, BF16>(a, s);
  return by_g<F32, F32>(a, s);
}

}  // namespace kvlr
