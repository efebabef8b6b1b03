// Append-side encode of new keys and values into the paged latent cache.
//
// BasisKV: Value Latents for Communication and Key Routing, English abstract:
// keys and values are compressed on write by low-rank projections; the value
// latent is stored, and what it cannot predict of the key is kept as a
// key-specific residual latent next to the original key.
//   v = RNE(V A_v)
//   routed: c = RNE((K - v W_pred) A_k), original key copied to its page
//   dense:  k = RNE(K A_k)
// These are true dense contractions and run on the matrix cores
// (bf16: v_mfma_f32_16x16x32_bf16; f32: v_mfma_f32_16x16x4_f32) with float32
// accumulation. The routed residual is evaluated as
//   c = K A_k + v (-(W_pred A_k)),
// an exact reassociation of the definition: the r_v x r_k matrix
// W_pred A_k is formed on the matrix cores, negated and, for bf16, split
// into a high and a low bf16 part so the product with the stored (bf16)
// latent v keeps about 16 significant bits of the matrix. It depends on the
// factors only: a preparation launch (one workgroup per KV head, the same
// code) can write it once in the B-operand layout the encode reads, and the
// encode then copies it instead of forming it in every workgroup.
//
// Work split: grid (KV head, token-tile groups). A workgroup stages the
// factor fragments of its head in LDS once, then loops over 64-token tiles,
// 16 tokens per wave: the wave loads its tokens' rows straight into MFMA
// A-operand registers, multiplies and rounds into its rows of the LDS tiles.
// With bf16 inputs the whole tile is then written column by column (each
// wave takes every fourth chunk column of the pages, one token per lane, so
// a store covers up to 64 consecutive slots); with f32 inputs each wave
// writes its own tokens' chunks. With FP8 latents (bf16 inputs and
// factors) the latents are rounded once from the float32 products to E4M3
// (nearest even, saturating at +-448) and stored as 8-byte chunks; the
// residual is taken against that stored latent, decoded exactly to bf16.
// A launch may also carry the step's query projection: its first grid rows
// then compute 16 x 16 tiles of q_proj (one per wave, on the float32 matrix
// cores), independent of the encode, which saves the projection's own launch.

#include "kvlr_device.h"
#include "kvlr_gemm_tile.h"
#include "kvlr_internal.h"

#ifndef KVLR_ENCODE_WGS
#define KVLR_ENCODE_WGS 0  // workgroups over all KV heads; 0: as many as stay resident at once
#endif

namespace kvlr {
namespace {


constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <class S>
struct Mma;

template <>
struct Mma<BF16> {
  static constexpr int KSTEP = 32;  // k per instruction
  static constexpr int KPL = 8;     // k elements per lane
  using E = uint16_t;
  using frag_t = bf16x8;
  __device__ static f32x4 mma(frag_t a, frag_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static frag_t lds(const E* p) {
    return __builtin_bit_cast(frag_t, *reinterpret_cast<const uint4*>(p));
  }
  __device__ static frag_t gmem(const uint8_t* p) { return __builtin_bit_cast(frag_t, load16(p)); }
  __device__ static frag_t zero() { return __builtin_bit_cast(frag_t, make_uint4(0, 0, 0, 0)); }
  __device__ static E store(float f) { return static_cast<E>(f32_to_bf16_rne(f)); }
  __device__ static float value(E e) { return __uint_as_float(static_cast<uint32_t>(e) << 16); }
};

template <>
struct Mma<F32> {
  static constexpr int KSTEP = 4;
  static constexpr int KPL = 1;
  using E = float;
  using frag_t = float;
  __device__ static f32x4 mma(frag_t a, frag_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static frag_t lds(const E* p) { return *p; }
  __device__ static frag_t gmem(const uint8_t* p) { return *reinterpret_cast<const float*>(p); }
  __device__ static frag_t zero() { return 0.f; }
  __device__ static E store(float f) { return f; }
  __device__ static float value(E e) { return e; }
};

// How rounded latents are held and stored: in the storage type S itself, or
// (LS = FP8, with S = BF16) as E4M3 codes rounded once from the float32
// products; the stored value latent is also the routed residual's operand.
template <class S, class LS>
struct Lat {
  using MM = Mma<S>;
  using E = typename MM::E;
  static constexpr int CB = 16;
  __device__ static E round(float f) { return MM::store(f); }
  __device__ static typename MM::frag_t frag(const E* p) { return MM::lds(p); }
  __device__ static void store_chunk(uint8_t* dst, const E* src) {
    store16(dst, *reinterpret_cast<const uint4*>(src));
  }
};
template <>
struct Lat<BF16, FP8> {
  using E = uint8_t;
  static constexpr int CB = 8;
  __device__ static E round(float f) { return static_cast<E>(f32_to_fp8_rne_sat(f)); }
  __device__ static bf16x8 frag(const E* p) { return FP8::to_bf16x8(*reinterpret_cast<const uint2*>(p)); }
  __device__ static void store_chunk(uint8_t* dst, const E* src) {
    *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
  }
};

template <class S, class LS, int D, int RV, int RK, bool ROUTED>
struct EncSmem {
  using MM = Mma<S>;
  using E = typename MM::E;
  using LE = typename Lat<S, LS>::E;
  static constexpr int KSTEP = MM::KSTEP, KPL = MM::KPL, CH = S::CH;
  static constexpr int KSD = D / KSTEP;                    // k-steps over head_dim
  static constexpr int KSV = (RV + KSTEP - 1) / KSTEP;     // k-steps over rank_v (zero padded)
  // B-operand fragments: [k-step][n-tile][lane][KPL]
  alignas(16) E av[KSD][RV / 16][kWave][KPL];
  alignas(16) E ak[KSD][RK / 16][kWave][KPL];
  alignas(16) E mhi[ROUTED ? KSV : 1][RK / 16][kWave][KPL];
  alignas(16) E mlo[(ROUTED && KPL > 1) ? KSV : 1][RK / 16][kWave][KPL];
  struct Tiles {
    // per-wave row-major tiles of the rounded latents (16 tokens each; read
    // across the waves as one 64-token tile)
    alignas(16) LE vt[kWaves][16][RV + CH];
    alignas(16) LE ct[kWaves][16][RK + CH];
  };
  // bf16: the tile's original keys, one 16-byte chunk per entry (64 tokens;
  // one spare entry per row keeps rows on rotating banks). Kept apart from
  // the latent tiles, so all of a tile's stores go out as one batch.
  static constexpr int KT_COLS = (KPL == CH) ? D / CH + 1 : 1;
  union {
    float mstage[ROUTED ? RV : 1][RK + 1];  // set-up only
    Tiles t;
  } u;
  uint4 kt[(KPL == CH && ROUTED) ? 64 : 1][KT_COLS];
  int tok_page[64];  // physical page of each token of the tile, -1 past the end
  int tok_slot[64];  // its slot in the page
};

__device__ inline void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Workgroup barrier for LDS hand-offs only: global stores already issued
// stay in flight across it.
__device__ inline void block_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Query-projection tiles carried by the same launch (kvlr_append_encode_project):
// the first qy grid rows hold them, one 16 x 16 tile of q_proj per wave; the
// encode's tile groups follow. qy = 0: none.
struct QTiles {
  const uint8_t* B_k;
  const float* q;
  float* q_proj;
  int batch, Hq, G, row_tiles, col_tiles, qy;
};

// The prepared residual operand -(W_pred A_k): per KV head its high parts,
// then (bf16) its low parts, each [k-step][n-tile][lane][KPL] as in EncSmem.
// out set: form it and write it (no tokens); in set: copy it, do not form it.
struct MPrep {
  const uint8_t* in;
  uint8_t* out;
};

template <class S, int RV, int RK>
constexpr size_t mprep_head_bytes() {
  using MM = Mma<S>;
  constexpr int KSV = (RV + MM::KSTEP - 1) / MM::KSTEP;
  return static_cast<size_t>(KSV) * (RK / 16) * kWave * MM::KPL * sizeof(typename MM::E) *
         (MM::KPL > 1 ? 2 : 1);
}

template <class S, class LS, int D, int RV, int RK, bool ROUTED>
__global__ __launch_bounds__(kThreads) void encode_kernel(
    const uint8_t* __restrict__ A_v, const uint8_t* __restrict__ A_k,
    const uint8_t* __restrict__ W_pred, const uint8_t* __restrict__ k_new,
    const uint8_t* __restrict__ v_new, const int32_t* __restrict__ cu_new,
    const int32_t* __restrict__ lens_before, const int32_t* __restrict__ page_table,
    uint8_t* __restrict__ v_lat, uint8_t* __restrict__ k_lat, uint8_t* __restrict__ k_exact,
    int Hkv, int P, int log2P, int max_pages, int batch, int total_new, KLayout kl, QTiles qt,
    MPrep mp) {
  using MM = Mma<S>;
  using SM = EncSmem<S, LS, D, RV, RK, ROUTED>;
  using LT = Lat<S, LS>;
  using E = typename MM::E;
  using LE = typename LT::E;
  using frag_t = typename MM::frag_t;
  constexpr int KSTEP = MM::KSTEP, KPL = MM::KPL, CH = S::CH, EB = S::ELEM_BYTES;
  constexpr int KSD = SM::KSD, KSV = SM::KSV;
  constexpr int NTV = RV / 16, NTK = RK / 16;
  constexpr int CV = RV / CH, CK = RK / CH, CD = D / CH;
  __shared__ SM sm;
  // cu_new[0 .. batch] at s_seq[0 ..], lens_before[0 .. batch) at s_seq[nb1 ..]
  extern __shared__ int s_seq[];
  const int nb1 = batch + 1 > kThreads ? batch + 1 : kThreads;

  if (static_cast<int>(blockIdx.y) < qt.qy) {  // a workgroup of query-projection tiles
    // grid column x holds KV head x's tiles, as it holds that head's encode
    // workgroups: workgroups go to the XCDs round robin by linear id, so with
    // H_kv = 8 columns every workgroup of a head shares one XCD's L2, and the
    // head's query rows and factor columns are fetched from memory once
    const int hg = blockIdx.x;
    const int t = static_cast<int>(blockIdx.y) * kWaves + static_cast<int>(threadIdx.x) / kWave;
    if (t < qt.row_tiles * qt.col_tiles) {
      const int ct = t / qt.row_tiles;
      qproj_tile<S, D>(W_pred, qt.B_k, qt.q, qt.q_proj, qt.batch, qt.Hq, qt.G, RV, RK, ROUTED ? 1 : 0,
                       t - ct * qt.row_tiles, ct, hg);
    }
    return;
  }
  // KV heads vary fastest over the grid: workgroups launched together take
  // the same tokens of every head, so the new rows (all heads of a token are
  // adjacent) and the pages written are read and written in whole spans
  const int g = blockIdx.x;
  const int tile0 = static_cast<int>(blockIdx.y) - qt.qy;
  const int tile_step = static_cast<int>(gridDim.y) - qt.qy;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const E* Av = reinterpret_cast<const E*>(A_v) + static_cast<size_t>(g) * D * RV;
  const E* Ak = reinterpret_cast<const E*>(A_k) + static_cast<size_t>(g) * D * RK;

  const int ntiles = (total_new + 63) / 64;
  const int r = lane & 15;        // A-operand row (token) of this lane
  const int kq = lane >> 4;       // A-operand k group of this lane
  // with 16-byte fragments (bf16) the key fragments are also the 16-byte
  // chunks of the original key and are stored from registers
  constexpr bool FRAG_IS_CHUNK = (KPL == CH);
  // Loads are unconditional (no branch around them): lanes past the last
  // token read token 0 instead, and since an output row of the products
  // depends only on its own token row, those rows are simply never stored.
  auto load_tile = [&](int tile, frag_t (&vf)[KSD], frag_t (&kf)[KSD]) {
    const int i = tile * 64 + wave * 16 + r;
    const size_t row_off = (static_cast<size_t>(i < total_new ? i : 0) * Hkv + g) * D * EB;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) vf[ks] = MM::gmem(v_new + row_off + (ks * KSTEP + KPL * kq) * EB);
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) kf[ks] = MM::gmem(k_new + row_off + (ks * KSTEP + KPL * kq) * EB);
  };
  constexpr int MT = ROUTED ? (NTV * NTK + kWaves - 1) / kWaves : 0;  // M tiles per wave
  frag_t wa[MT > 0 ? MT : 1][KSD];
  // the W_pred rows of this wave's tiles of M = W_pred A_k
  auto load_w = [&] {
    const uint8_t* Wg = W_pred + static_cast<size_t>(g) * RV * D * EB;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int ti = wave + m * kWaves;
      const int mt = (ti < NTV * NTK ? ti : 0) / NTK;
      const int row = mt * 16 + (lane & 15);
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks)
        wa[m][ks] = MM::gmem(Wg + (static_cast<size_t>(row) * D + ks * KSTEP + KPL * (lane >> 4)) * EB);
    }
  };
  // M's tiles on the matrix cores (A_k's fragments staged in LDS), then
  // -M split into the high and low B-operand fragments of the residual
  // products; ends with the workgroup synchronised
  auto form_m = [&] {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int ti = wave + m * kWaves;
      if (ti >= NTV * NTK) continue;
      const int mt = ti / NTK, nt = ti - mt * NTK;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) acc = MM::mma(wa[m][ks], MM::lds(&sm.ak[ks][nt][lane][0]), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.u.mstage[mt * 16 + 4 * (lane >> 4) + i][nt * 16 + (lane & 15)] = acc[i];
    }
    __syncthreads();
    for (int idx = tid; idx < KSV * NTK * kWave * KPL; idx += kThreads) {
      const int e = idx % KPL, l = (idx / KPL) % kWave, nt = (idx / (KPL * kWave)) % NTK;
      const int ks = idx / (KPL * kWave * NTK);
      const int k = ks * KSTEP + KPL * (l >> 4) + e, n = nt * 16 + (l & 15);
      const float mv = (k < RV) ? -sm.u.mstage[k][n] : 0.f;
      const E hi = MM::store(mv);
      sm.mhi[ks][nt][l][e] = hi;
      if constexpr (KPL > 1) sm.mlo[ks][nt][l][e] = MM::store(mv - MM::value(hi));
    }
    __syncthreads();
  };
  constexpr size_t kMHalf = static_cast<size_t>(KSV) * NTK * kWave * KPL * sizeof(E);
  constexpr size_t kMHead = mprep_head_bytes<S, RV, RK>();
  static_assert(kMHead == kMHalf * (KPL > 1 ? 2 : 1), "prepared operand size");

  // ---- stage B fragments: element (k, n) with k = ks*KSTEP + KPL*(l/16) + e,
  // n = nt*16 + l%16; each thread reads CH consecutive n of one row k
  auto stage = [&](const E* src, E* dst, auto rr) {
    constexpr int R = decltype(rr)::value;
    constexpr int RC = R / CH;                    // chunks per row
    constexpr int NCHK = D * RC;                  // chunks of the factor
    constexpr int IT = (NCHK + kThreads - 1) / kThreads;
    uint4 buf[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {             // every load in flight first
      const int idx = tid + it * kThreads;
      const int k = idx / RC, n0 = (idx - k * RC) * CH;
      buf[it] = (idx < NCHK) ? load16(src + static_cast<size_t>(k) * R + n0) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = tid + it * kThreads;
      if (idx >= NCHK) continue;
      const int k = idx / RC, n0 = (idx - k * RC) * CH;
      float x[CH];
      S::unpack(buf[it], x);
      const int ks = k / KSTEP, kk = k - ks * KSTEP;
#pragma unroll
      for (int e2 = 0; e2 < CH; ++e2) {
        const int n = n0 + e2;
        const int l = (kk / KPL) * 16 + (n & 15);
        dst[((static_cast<size_t>(ks) * (R / 16) + (n >> 4)) * kWave + l) * KPL + (kk % KPL)] =
            MM::store(x[e2]);
      }
    }
  };
  if constexpr (ROUTED) {
    if (mp.out) {  // preparation launch: form -M once and write it out
      load_w();
      stage(Ak, &sm.ak[0][0][0][0], std::integral_constant<int, RK>{});
      __syncthreads();
      form_m();
      uint8_t* dst = mp.out + static_cast<size_t>(g) * kMHead;
      for (size_t o = static_cast<size_t>(tid) * 16; o < kMHalf; o += kThreads * 16) {
        store16(dst + o, *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(&sm.mhi[0][0][0][0]) + o));
        if constexpr (KPL > 1)
          store16(dst + kMHalf + o,
                  *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(&sm.mlo[0][0][0][0]) + o));
      }
      return;
    }
  }
  // each thread's entries of cu_new and lens_before (clamped indexes: every
  // thread reads and later stores, so the requests are not deferred), this
  // workgroup's first tile, and the W_pred rows of M (unless it comes
  // prepared), are requested before the set-up below
  const int cu_first = cu_new[tid <= batch ? tid : batch];
  const int lb_first = lens_before[tid < batch ? tid : batch - 1];
  frag_t vf[KSD], kf[KSD];
  load_tile(tile0, vf, kf);
  if constexpr (ROUTED) {
    if (!mp.in) load_w();
  }
  stage(Av, &sm.av[0][0][0][0], std::integral_constant<int, RV>{});
  stage(Ak, &sm.ak[0][0][0][0], std::integral_constant<int, RK>{});
  if constexpr (ROUTED) {
    if (mp.in) {  // the prepared -M, copied into its LDS fragments
      const uint8_t* src = mp.in + static_cast<size_t>(g) * kMHead;
      for (size_t o = static_cast<size_t>(tid) * 16; o < kMHalf; o += kThreads * 16) {
        *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(&sm.mhi[0][0][0][0]) + o) = load16(src + o);
        if constexpr (KPL > 1)
          *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(&sm.mlo[0][0][0][0]) + o) =
              load16(src + kMHalf + o);
      }
    }
  }
  s_seq[tid] = cu_first;
  s_seq[nb1 + tid] = lb_first;
  for (int b = tid + kThreads; b <= batch; b += kThreads) s_seq[b] = cu_new[b];
  for (int b = tid + kThreads; b < batch; b += kThreads) s_seq[nb1 + b] = lens_before[b];
  __syncthreads();

  // sequence of token i: largest b with cu_new[b] <= i (offsets staged in LDS);
  // returns its physical page and the token's slot in the page, or -1 past
  // the last token or past the end of its page-table row (the entry read
  // then is entry 0 of sequence 0, and not used); a negative entry also
  // gives -1, so such a token is not stored
  auto locate = [&](int tile, size_t& slot_off) -> int {
    const int i = tile * 64 + wave * 16 + r;
    slot_off = 0;
    const int32_t* e = page_table;
    bool ok = false;
    if (i < total_new) {
      int lo = 0, hi = batch;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_seq[mid] <= i) lo = mid; else hi = mid;
      }
      const int pos = s_seq[nb1 + lo] + (i - s_seq[lo]);
      slot_off = static_cast<size_t>(pos & (P - 1));
      ok = pos >= 0 && (pos >> log2P) < max_pages;
      if (ok) e = page_table + static_cast<size_t>(lo) * max_pages + (pos >> log2P);
    }
    const int v = *e;
    return ok ? v : -1;
  };
  // the first tile's page-table entry is requested before M is formed
  size_t slot0 = 0;
  const int phys0 = locate(tile0, slot0);

  if constexpr (ROUTED) {
    if (!mp.in) form_m();  // M = W_pred A_k [RV x RK], 16x16 tiles spread over the waves
  }

  // v = V A_v and the residual (routed) or key latent (dense), rounded into
  // the wave's rows of the LDS tiles; `after_v` runs once the v rows are
  // written (the routed residual reads them back)
  auto products = [&](const frag_t (&vf)[KSD], const frag_t (&kf)[KSD], auto after_v) {
    f32x4 vacc[NTV];
#pragma unroll
    for (int nt = 0; nt < NTV; ++nt) vacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) vacc[nt] = MM::mma(vf[ks], MM::lds(&sm.av[ks][nt][lane][0]), vacc[nt]);
#pragma unroll
    for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.u.t.vt[wave][4 * kq + j][nt * 16 + r] = LT::round(vacc[nt][j]);
    f32x4 cacc[NTK];
#pragma unroll
    for (int nt = 0; nt < NTK; ++nt) cacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
      for (int nt = 0; nt < NTK; ++nt) cacc[nt] = MM::mma(kf[ks], MM::lds(&sm.ak[ks][nt][lane][0]), cacc[nt]);
    wave_lds_sync();
    after_v();
    if constexpr (ROUTED) {
#pragma unroll
      for (int ks = 0; ks < KSV; ++ks) {
        const int k = ks * KSTEP + KPL * kq;
        const frag_t a = (k < RV) ? LT::frag(&sm.u.t.vt[wave][r][k]) : MM::zero();
#pragma unroll
        for (int nt = 0; nt < NTK; ++nt) {
          cacc[nt] = MM::mma(a, MM::lds(&sm.mhi[ks][nt][lane][0]), cacc[nt]);
          if constexpr (KPL > 1) cacc[nt] = MM::mma(a, MM::lds(&sm.mlo[ks][nt][lane][0]), cacc[nt]);
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < NTK; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.u.t.ct[wave][4 * kq + j][nt * 16 + r] = LT::round(cacc[nt][j]);
    wave_lds_sync();
  };
  // per-head residual ranks: head g keeps its first ckg chunks, at its own
  // offset in the page
  const int ckg = kl.adaptive ? kl.ck[g] : CK;
  const size_t kpage = kl.adaptive ? static_cast<size_t>(kl.page_chunks) : static_cast<size_t>(Hkv) * CK;
  const size_t koff = kl.adaptive ? static_cast<size_t>(kl.off[g]) : static_cast<size_t>(g) * CK;

  // one tile, bf16 storage: the workgroup gathers the tile's 64 tokens in
  // LDS, then each wave writes whole chunk columns of the pages (a column is
  // P consecutive slots, so a store instruction covers up to 64 slots: 1 KB
  // of bf16, 512 bytes of FP8), taking every fourth column. The original
  // keys and the latents go out together after the products: the in-order
  // memory counter then waits for a tile's stores once, not per phase.
  auto process_cols = [&](int tile, const frag_t (&vf)[KSD], const frag_t (&kf)[KSD], int phys,
                          size_t slot_off) {
    const int i = tile * 64 + wave * 16 + r;
    const bool valid = i < total_new;
    const int t_own = wave * 16 + r;  // this lane's token within the tile
    if constexpr (ROUTED && FRAG_IS_CHUNK) {
      // fragment ks of this lane is chunk ks * KSTEP / CH + kq of the key row
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks)
        sm.kt[t_own][ks * (KSTEP / CH) + kq] = __builtin_bit_cast(uint4, kf[ks]);
    }
    // the products use only this wave's rows; the token's page (its lookup
    // still in flight) is needed only by the stores after the barrier
    products(vf, kf, [] {});
    if (kq == 0) {
      sm.tok_page[t_own] = (valid && phys >= 0) ? phys : -1;
      sm.tok_slot[t_own] = static_cast<int>(slot_off);
    }
    block_lds_sync();
    const int pg = sm.tok_page[lane];  // lane = token of the tile from here on
    const size_t slot = static_cast<size_t>(sm.tok_slot[lane]);
    if constexpr (ROUTED && FRAG_IS_CHUNK) {
      constexpr int NCOL = CD / kWaves;  // key chunk columns per wave
      static_assert(CD % kWaves == 0, "key chunk columns split evenly over the waves");
      if (pg >= 0) {
        uint8_t* kd = k_exact + (static_cast<size_t>(pg) * Hkv + g) * CD * P * 16 + slot * 16;
#pragma unroll
        for (int j = 0; j < NCOL; ++j)
          store16(kd + static_cast<size_t>(wave + j * kWaves) * P * 16, sm.kt[lane][wave + j * kWaves]);
      }
    }
    if (pg >= 0) {
      const LE* vrow = &sm.u.t.vt[0][0][0] + lane * (RV + CH);
      const LE* crow = &sm.u.t.ct[0][0][0] + lane * (RK + CH);
      uint8_t* vd = v_lat + (static_cast<size_t>(pg) * Hkv + g) * CV * P * LT::CB + slot * LT::CB;
      uint8_t* cd = k_lat + (static_cast<size_t>(pg) * kpage + koff) * P * LT::CB + slot * LT::CB;
#pragma unroll
      for (int c = wave; c < CV; c += kWaves) LT::store_chunk(vd + static_cast<size_t>(c) * P * LT::CB, vrow + c * CH);
#pragma unroll
      for (int c = wave; c < CK; c += kWaves)
        if (c < ckg) LT::store_chunk(cd + static_cast<size_t>(c) * P * LT::CB, crow + c * CH);
    }
    block_lds_sync();  // the next tile rewrites the tiles and locations
  };

  // one tile, f32 storage: each wave stores its 16 tokens' chunks
  auto process_rows = [&](int tile, const frag_t (&vf)[KSD], const frag_t (&kf)[KSD], int phys_id,
                          size_t slot_off) {
    const int i = tile * 64 + wave * 16 + r;
    const bool valid = i < total_new && phys_id >= 0;
    const size_t phys = static_cast<size_t>(valid ? phys_id : 0);
    if constexpr (ROUTED) {
      if (valid) {
        uint8_t* kd = k_exact + (phys * Hkv + g) * CD * P * 16 + slot_off * 16;
        const size_t row_off = (static_cast<size_t>(i) * Hkv + g) * D * EB;
        for (int c = kq; c < CD; c += 4)
          store16(kd + static_cast<size_t>(c) * P * 16, load16(k_new + row_off + c * 16));
      }
    }
    products(vf, kf, [&] {
      if (valid) {
        uint8_t* dst = v_lat + (phys * Hkv + g) * CV * P * LT::CB + slot_off * LT::CB;
#pragma unroll
        for (int c0 = 0; c0 < CV; c0 += 4) {
          const int c = c0 + kq;
          if (c < CV) LT::store_chunk(dst + static_cast<size_t>(c) * P * LT::CB, &sm.u.t.vt[wave][r][c * CH]);
        }
      }
    });
    if (valid) {
      uint8_t* dst = k_lat + (phys * kpage + koff) * P * LT::CB + slot_off * LT::CB;
#pragma unroll
      for (int c0 = 0; c0 < CK; c0 += 4) {
        const int c = c0 + kq;
        if (c < ckg) LT::store_chunk(dst + static_cast<size_t>(c) * P * LT::CB, &sm.u.t.ct[wave][r][c * CH]);
      }
    }
    wave_lds_sync();
  };
  auto process = [&](int tile, const frag_t (&vf)[KSD], const frag_t (&kf)[KSD], int phys,
                     size_t slot_off) {
    if constexpr (FRAG_IS_CHUNK) process_cols(tile, vf, kf, phys, slot_off);
    else process_rows(tile, vf, kf, phys, slot_off);
  };

  for (int tile = tile0; tile < ntiles; tile += tile_step) {
    size_t slot = slot0;
    int phys = phys0;
    if (tile != tile0) {
      load_tile(tile, vf, kf);
      phys = locate(tile, slot);
    }
    process(tile, vf, kf, phys, slot);
  }
}

template <class S, class LS, int D, int RV, int RK, bool ROUTED>
hipError_t launch_t(const EncodeArgs& a, hipStream_t s) {
  const int log2P = __builtin_ctz(static_cast<unsigned>(a.dm.P));
  const int ntiles = (a.total_new + 63) / 64;
  const size_t lds = 2 * static_cast<size_t>(a.batch + 1 > kThreads ? a.batch + 1 : kThreads) * sizeof(int);
  // A persistent grid: the workgroups that fit on the device at once, each
  // looping over tiles (a second, partial round of workgroups left most of
  // the device idle behind it, and fewer, longer-lived workgroups stage the
  // factors fewer times).
  int wgs = KVLR_ENCODE_WGS;
  if (wgs <= 0) {
    int per_cu = 0, dev = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, encode_kernel<S, LS, D, RV, RK, ROUTED>,
                                                     kThreads, lds) != hipSuccess ||
        hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipGetLastError();
    wgs = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  }
  int per_head = (wgs + a.dm.Hkv - 1) / a.dm.Hkv;
  if (per_head > ntiles) per_head = ntiles;
  QTiles qt{};
  if (a.q) {
    qt.B_k = static_cast<const uint8_t*>(a.B_k);
    qt.q = a.q;
    qt.q_proj = a.q_proj;
    qt.batch = a.batch;
    qt.Hq = a.dm.Hq;
    qt.G = a.dm.G;
    qt.row_tiles = (a.batch * a.dm.G + 15) / 16;
    qt.col_tiles = ((ROUTED ? RV : 0) + RK) / 16;
    qt.qy = (qt.row_tiles * qt.col_tiles + kWaves - 1) / kWaves;  // rows of tiles per head
  }
  if (per_head + qt.qy == 0) return hipSuccess;
  dim3 grid(a.dm.Hkv, per_head + qt.qy);
  hipLaunchKernelGGL((encode_kernel<S, LS, D, RV, RK, ROUTED>), grid, dim3(kThreads), lds, s,
                     static_cast<const uint8_t*>(a.A_v), static_cast<const uint8_t*>(a.A_k),
                     static_cast<const uint8_t*>(a.W_pred), static_cast<const uint8_t*>(a.k_new),
                     static_cast<const uint8_t*>(a.v_new), a.cu_new, a.lens_before, a.page_table,
                     static_cast<uint8_t*>(a.v_lat), static_cast<uint8_t*>(a.k_lat),
                     static_cast<uint8_t*>(a.k_exact), a.dm.Hkv, a.dm.P, log2P, a.max_pages,
                     a.batch, a.total_new, a.kl, qt,
                     MPrep{ROUTED ? static_cast<const uint8_t*>(a.m_prep) : nullptr, nullptr});
  return hipGetLastError();
}

// The preparation launch: one workgroup per KV head writes its -M.
template <class S, class LS, int D, int RV, int RK, bool ROUTED>
hipError_t launch_prep_t(const EncodeArgs& a, void* out, hipStream_t s) {
  if constexpr (!ROUTED) {
    return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((encode_kernel<S, LS, D, RV, RK, ROUTED>), dim3(a.dm.Hkv, 1), dim3(kThreads),
                       sizeof(int), s, static_cast<const uint8_t*>(a.A_v),
                       static_cast<const uint8_t*>(a.A_k), static_cast<const uint8_t*>(a.W_pred),
                       nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                       a.dm.Hkv, a.dm.P, 0, 1, 0, 0, a.kl, QTiles{},
                       MPrep{nullptr, static_cast<uint8_t*>(out)});
    return hipGetLastError();
  }
}

// What the dispatch below does per instance: launch the encode, launch the
// preparation, or report the prepared operand's bytes.
struct EncodeOp {
  enum Kind { kEncode, kPrep, kBytes } kind;
  void* out;
  size_t* bytes;
};

template <class S, class LS, int D, int RV, int RK>
hipError_t by_mode(const EncodeArgs& a, const EncodeOp& op, hipStream_t s) {
  if (op.kind == EncodeOp::kBytes) {
    *op.bytes = a.dm.exact ? mprep_head_bytes<S, RV, RK>() * a.dm.Hkv : 0;
    return hipSuccess;
  }
  if (op.kind == EncodeOp::kPrep)
    return a.dm.exact ? launch_prep_t<S, LS, D, RV, RK, true>(a, op.out, s) : hipErrorInvalidValue;
  return a.dm.exact ? launch_t<S, LS, D, RV, RK, true>(a, s) : launch_t<S, LS, D, RV, RK, false>(a, s);
}

template <class S, class LS, int D, int RV>
hipError_t by_rk(const EncodeArgs& a, const EncodeOp& op, hipStream_t s) {
  switch (a.dm.RK) {
    case 16: return by_mode<S, LS, D, RV, 16>(a, op, s);
    case 32: return by_mode<S, LS, D, RV, 32>(a, op, s);
    case 64: return by_mode<S, LS, D, RV, 64>(a, op, s);
  }
  return hipErrorInvalidValue;
}

template <class S, class LS, int D>
hipError_t by_rv(const EncodeArgs& a, const EncodeOp& op, hipStream_t s) {
  switch (a.dm.RV) {
    case 16: return by_rk<S, LS, D, 16>(a, op, s);
    case 32: return by_rk<S, LS, D, 32>(a, op, s);
    case 64: return by_rk<S, LS, D, 64>(a, op, s);
    case 128:
      // full-width values: bf16 storage only (the f32 tiles would not fit in LDS)
      if constexpr (D == 128 && S::CH == 8 && LS::CB == 16) return by_rk<S, LS, D, 128>(a, op, s);
      break;
  }
  return hipErrorInvalidValue;
}

template <class S, class LS>
hipError_t by_d(const EncodeArgs& a, const EncodeOp& op, hipStream_t s) {
  switch (a.dm.D) {
    case 64: return by_rv<S, LS, 64>(a, op, s);
    case 128: return by_rv<S, LS, 128>(a, op, s);
  }
  return hipErrorInvalidValue;
}

hipError_t dispatch(const EncodeArgs& a, const EncodeOp& op, hipStream_t s) {
  if (a.dm.lat == 2) return by_d<BF16, FP8>(a, op, s);
  if (a.dm.dtype == 0) return by_d<BF16, BF16>(a, op, s);
  return by_d<F32, F32>(a, op, s);
}

}  // namespace

hipError_t launch_encode(const EncodeArgs& a, hipStream_t s) {
  if (a.batch == 0 || (a.total_new == 0 && !a.q)) return hipSuccess;
  return dispatch(a, EncodeOp{EncodeOp::kEncode, nullptr, nullptr}, s);
}

hipError_t launch_encode_prep(const EncodeArgs& a, void* out, hipStream_t s) {
  return dispatch(a, EncodeOp{EncodeOp::kPrep, out, nullptr}, s);
}

size_t encode_prep_bytes(const Dims& dm) {
  EncodeArgs a{};
  a.dm = dm;
  size_t bytes = 0;
  if (dispatch(a, EncodeOp{EncodeOp::kBytes, nullptr, &bytes}, nullptr) != hipSuccess) return 0;
  return bytes;
}

}  // namespace kvlr
