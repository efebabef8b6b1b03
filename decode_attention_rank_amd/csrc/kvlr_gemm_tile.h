// Small dense products on the float32 matrix cores, shared by the query
// projection and up-projection kernels and by the encode launch that also
// projects the step's queries.
//
// BasisKV: Value Latents for Communication and Key Routing, English abstract:
// scoring against latents needs the query mapped through the factors
// (q_hat = q W_pred^T, q_tilde = q B_k^T), and the decoder B_v is applied once
// per query head to z.
#pragma once

#include "kvlr_device.h"

namespace kvlr {

// One 16 x 16 output tile of  out[r, n] = sum_k a[r, k] w(k, n)  on the float32
// matrix cores (v_mfma_f32_16x16x4_f32), one wave per tile. Rows r are the
// (sequence, query head) rows of one KV group: r = b * G + (h - g * G).
// Lane l feeds A[l % 16][k] and B[k][l % 16] with k taken from the contiguous
// quarter (l / 16) * K/4 .. + K/4 of the reduction, so every operand of the
// tile is loaded before the first multiply and the loads overlap.
// W_NMAJOR: w(k, n) = W[n][k] (rows of W are outputs), else W[k][n].
template <class S, int K, bool W_NMAJOR>
__device__ inline void small_gemm_tile(const float* __restrict__ a_src, int a_row_stride,
                                       const uint8_t* __restrict__ W, int w_ld, int rows,
                                       int row_tile, int n0, int G, int Hq, int g,
                                       float* __restrict__ out, int out_stride, int out_off) {
  constexpr int KQ = K / 4;  // reduction elements per lane quarter
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  const int kq = lane >> 4;
  const int ra = row_tile * 16 + j;
  const bool va = ra < rows;
  const int ba = va ? ra / G : 0;
  const int ha = va ? g * G + (ra - ba * G) : 0;
  float av[KQ], bv[KQ];
  const float* ar = a_src + static_cast<size_t>(ba * Hq + ha) * a_row_stride + kq * KQ;
#pragma unroll
  for (int i = 0; i < KQ; i += 4) {
    const float4 t = va ? *reinterpret_cast<const float4*>(ar + i) : make_float4(0.f, 0.f, 0.f, 0.f);
    av[i] = t.x;
    av[i + 1] = t.y;
    av[i + 2] = t.z;
    av[i + 3] = t.w;
  }
  if constexpr (W_NMAJOR) {
    constexpr int CH = S::CH;
    const uint8_t* wr = W + (static_cast<size_t>(n0 + j) * w_ld + kq * KQ) * S::ELEM_BYTES;
#pragma unroll
    for (int c = 0; c < KQ / CH; ++c) {
      float x[CH];
      S::unpack(load16(wr + c * 16), x);
#pragma unroll
      for (int e = 0; e < CH; ++e) bv[c * CH + e] = x[e];
    }
  } else {
#pragma unroll
    for (int i = 0; i < KQ; ++i)
      bv[i] = S::load1(W, static_cast<long>(kq * KQ + i) * w_ld + n0 + j);
  }
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < KQ; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[i], acc, 0, 0, 0);
  // result layout: lane holds rows 4 * (l / 16) + i of column l % 16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = row_tile * 16 + 4 * kq + i;
    if (r >= rows) continue;
    const int bb = r / G;
    const int hh = g * G + (r - bb * G);
    out[static_cast<size_t>(bb * Hq + hh) * out_stride + out_off + n0 + j] = acc[i];
  }
}

// One 16 x 16 tile of the query images: q_proj rows are
// [q W_pred^T (exact mode only), q B_k^T]; col_tile counts 16-column tiles
// across both parts, g is the KV head.
template <class S, int D>
__device__ inline void qproj_tile(const uint8_t* __restrict__ W_pred, const uint8_t* __restrict__ B_k,
                                  const float* __restrict__ q, float* __restrict__ q_proj, int B,
                                  int Hq, int G, int RV, int RK, int exact, int row_tile,
                                  int col_tile, int g) {
  const int RVe = exact ? RV : 0;
  const int Wd = RVe + RK;
  const int n0 = col_tile * 16;
  const bool pred = n0 < RVe;
  const uint8_t* W = pred ? W_pred + static_cast<size_t>(g) * RV * D * S::ELEM_BYTES
                          : B_k + static_cast<size_t>(g) * RK * D * S::ELEM_BYTES;
  const int wn0 = pred ? n0 : n0 - RVe;
  small_gemm_tile<S, D, true>(q, D, W, D, B * G, row_tile, wn0, G, Hq, g, q_proj, Wd,
                              pred ? 0 : RVe);
}

}  // namespace kvlr
