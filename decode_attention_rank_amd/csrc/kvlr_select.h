// Exact top-k page selection of one (sequence, KV head) pair in LDS, shared by
// the selection launch (one workgroup per pair) and the routing launch's
// ticket form (the pair's last chunk selects).
//
// BasisKV: Value Latents for Communication and Key Routing, English abstract:
// the approximate page scores decide which key pages are read. The kept set
// is the k largest scores, equal scores going to the lower page index, in
// ascending page order. Scores enter as order keys (a larger key is a larger
// score); a 4-pass radix select on 8-bit digits finds the k-th largest key,
// and an ascending compaction takes every larger key plus the lowest-index
// equal ones.
#pragma once

#include "kvlr_device.h"

namespace kvlr {

constexpr int kSelectLds = 4096;  // largest page count selected from LDS
constexpr int kSelectMaxWaves = 16;  // workgroups of up to 1024 threads

// LDS of one selection: the order keys of pages 0..N-1, the same pages'
// page-table entries (filled by callers that want physical pages), one
// 256-bin histogram per radix pass (lane l of a scan owns bins 4l..4l+3) and
// the block scan's per-wave slots.
struct SelectLds {
  uint32_t keys[kSelectLds];
  int32_t pt[kSelectLds];
  uint4 hist4[4][kWave];
  int lds4[kSelectMaxWaves];
};

// Exclusive prefix sum of v over the workgroup (NT threads) in thread order;
// also returns the total. Two barriers.
template <int NT>
__device__ inline int block_excl_sum(int v, int* total, int* lds4) {
  static_assert(NT % kWave == 0 && NT / kWave <= kSelectMaxWaves, "workgroup size");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) lds4[wave] = incl;
  __syncthreads();
  int before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    const int c = lds4[w];
    before += (w < wave) ? c : 0;
    sum += c;
  }
  __syncthreads();
  *total = sum;
  return before + incl - v;
}

// Clears the pass histograms; call before the barrier that publishes the keys.
__device__ inline void select_lds_clear(SelectLds& s) {
  if (threadIdx.x < 4 * kWave) (&s.hist4[0][0])[threadIdx.x] = make_uint4(0, 0, 0, 0);
}

// The k largest of s.keys[0..N) (N <= kSelectLds, keys published and the
// workgroup of NT threads synchronised, histograms cleared): emit(pos, j) is
// called once for each kept page j, pos being its rank in ascending page
// order (0..k-1).
// k >= N keeps every page, k <= 0 none. Every thread of the workgroup calls
// this; it contains barriers. Each pass has its own histogram, so a pass
// costs one barrier: after it every wave scans the histogram itself and finds
// the same bin. The passes stop early once the bin holding the k-th largest
// key is taken whole. The compaction gives thread t the contiguous pages
// t*per .. t*per+per-1, placed by one block-wide scan of the packed (above,
// equal) counts.
template <int NT, class Emit>
__device__ void select_keys_lds(SelectLds& s, int N, int k, Emit emit) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const bool take_all = (k >= N);
  // the kept pages: (key & pmask) > prefix, then the kk lowest-index pages
  // with (key & pmask) == prefix
  uint32_t prefix = 0, pmask = 0;
  int kk = k;
  if (!take_all && k > 0) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      uint32_t* h = reinterpret_cast<uint32_t*>(&s.hist4[pass][0]);
      for (int j = tid; j < N; j += NT) {
        const uint32_t key = s.keys[j];
        if ((key & pmask) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      // every wave: suffix sums from the top bin down, then the bin holding
      // the kk-th largest candidate (lane 0's suffix is every candidate, so
      // some lane qualifies)
      const uint4 hb = s.hist4[pass][lane];
      const uint32_t local = hb.x + hb.y + hb.z + hb.w;
      uint32_t suf = local;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t o = __shfl_down(suf, off, kWave);
        if (lane + off < kWave) suf += o;
      }
      const uint32_t need = static_cast<uint32_t>(kk);
      const int top = 63 - __clzll(__ballot(suf >= need));
      // bins 4l+3 .. 4l of lane l, scanned from the top
      const uint32_t a3 = suf - local, a2 = a3 + hb.w, a1 = a2 + hb.z, a0 = a1 + hb.y;
      const int d = (a3 + hb.w >= need) ? 3 : (a2 + hb.z >= need) ? 2 : (a1 + hb.y >= need) ? 1 : 0;
      const uint32_t above = (d == 3) ? a3 : (d == 2) ? a2 : (d == 1) ? a1 : a0;
      const uint32_t cnt = (d == 3) ? hb.w : (d == 2) ? hb.z : (d == 1) ? hb.y : hb.x;
      const uint32_t digit = static_cast<uint32_t>(__builtin_amdgcn_readlane(4 * lane + d, top));
      const int above_t = __builtin_amdgcn_readlane(static_cast<int>(above), top);
      const int cnt_t = __builtin_amdgcn_readlane(static_cast<int>(cnt), top);
      prefix |= digit << shift;
      pmask |= 255u << shift;
      kk -= above_t;
      if (cnt_t == kk) break;  // the whole bin is kept: the same in every wave
    }
  }
  const int per = (N + NT - 1) / NT;
  const int jb = min(tid * per, N), je = min(jb + per, N);
  const bool use_eq = !take_all && k > 0;
  int n_gt = 0, n_eq = 0;
  for (int j = jb; j < je; ++j) {
    const uint32_t key = s.keys[j] & pmask;
    n_gt += (take_all || key > prefix) ? 1 : 0;
    n_eq += (use_eq && key == prefix) ? 1 : 0;
  }
  // one scan of both counts (each sum is at most N <= 4096 < 2^16); the
  // equal keys are taken in index order, so the threads before this one
  // took min(kk, equal keys before) of them
  int tot = 0;
  const int packed = block_excl_sum<NT>((n_gt << 16) | n_eq, &tot, s.lds4);
  const int gt_before = packed >> 16, eq_before = packed & 0xffff;
  int pos = gt_before + min(kk, eq_before);
  int eq_rank = eq_before;
  for (int j = jb; j < je; ++j) {
    const uint32_t key = s.keys[j] & pmask;
    const bool gt = take_all || key > prefix;
    const bool eq = use_eq && key == prefix;
    const bool take = gt || (eq && eq_rank < kk);
    eq_rank += eq ? 1 : 0;
    if (take) {
      emit(pos, j);
      ++pos;
    }
  }
}

// Pages kept for a pair of n pages: the caller's per-sequence budget
// (clamped to [0, n]), else the fraction num/den rounded up and at least one
// page of a non-empty sequence; at most k_max.
__device__ inline int pages_to_keep(int n, const int32_t* k_pages, int b, int num, int den, int k_max) {
  if (n <= 0) return 0;
  int k;
  if (k_pages) {
    k = min(n, max(k_pages[b], 0));
  } else {
    const long long want = (static_cast<long long>(n) * num + den - 1) / den;
    k = static_cast<int>(min(static_cast<long long>(n), max(1LL, want)));
  }
  return min(k, k_max);
}

}  // namespace kvlr
