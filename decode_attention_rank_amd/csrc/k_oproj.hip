// Output projection seen from the value latents.
//
// BasisKV: Value Latents for Communication and Key Routing, English abstract
// and method details (key innovation): value compression is tied to the
// output projection. With o_h = z_h B_v[g(h)], the attention output through
// the output weight W_o ([hidden][H_q d], rows are output features) is
//   out = W_o concat_h(o_h) = F concat_h(z_h),  F = W_o blockdiag_h(B_v[g(h)]^T),
// F of shape [hidden][H_q r_v]: r_v instead of d inputs per head.
//
//  - fold_kernel forms F once (a weight preparation): per (16 output rows,
//    head) one wave multiplies W_o's head block by B_v^T on the matrix cores
//    (v_mfma_f32_16x16x32_bf16, both operands exact bf16, float32 sums) and
//    rounds F to bf16.
//  - oproj_kernel applies F to a batch of latent outputs: a skinny product
//    ([batch x H_q r_v] by [H_q r_v x hidden]) bound by reading F once. A
//    workgroup covers 16 or 32 output features; its 8 waves split the
//    reduction and request several k-steps of loads at a time. Each wave reads F rows as 16-byte
//    B fragments and the float32 latents as bf16 high and low halves (two
//    products per step); the partial tiles are summed through LDS in a
//    fixed order with two barriers.

#include "kvlr_device.h"
#include "kvlr_internal.h"

namespace kvlr {
namespace {


template <int D, int RV>
__global__ __launch_bounds__(kWave) void fold_kernel(const uint8_t* __restrict__ W_o,
                                                     const uint8_t* __restrict__ B_v,
                                                     uint16_t* __restrict__ F, int Hq, int G) {
  constexpr int KS = D / 32;   // k-steps over the head's d inputs
  constexpr int NT = RV / 16;  // 16-wide tiles of the head's latents
  const int lane = threadIdx.x;
  const int kq = lane >> 4, col = lane & 15;
  const int n0 = blockIdx.x * 16;
  const int h = blockIdx.y;
  const int g = h / G;
  const size_t ldw = static_cast<size_t>(Hq) * D;  // W_o row length (elements)
  bf16x8 a[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st)
    a[st] = __builtin_bit_cast(
        bf16x8, load16(W_o + ((n0 + col) * ldw + static_cast<size_t>(h) * D + st * 32 + kq * 8) * 2));
  const uint8_t* Bg = B_v + static_cast<size_t>(g) * RV * D * 2;
  const size_t ldf = static_cast<size_t>(Hq) * RV;  // F row length
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      // B[j][e] = B_v[g][e][j]: lane (e = t*16 + col, j = st*32 + kq*8 ..)
      const bf16x8 b = __builtin_bit_cast(
          bf16x8, load16(Bg + ((static_cast<size_t>(t) * 16 + col) * D + st * 32 + kq * 8) * 2));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[st], b, acc, 0, 0, 0);
    }
    // lane holds rows 4*kq + v (output features) of column col (latent e)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const size_t n = static_cast<size_t>(n0 + 4 * kq + v);
      F[n * ldf + static_cast<size_t>(h) * RV + t * 16 + col] =
          static_cast<uint16_t>(f32_to_bf16_rne(acc[v]));
    }
  }
}

constexpr int kOWaves = 8;                 // waves per workgroup (split reduction)
constexpr int kOThreads = kOWaves * kWave;
// MG: 16-row batch tiles per pass over F; kNT: 16-column output tiles per
// workgroup (more columns share each latent read); kUnroll: k-steps whose
// loads go out together. Measured best: (1, 1, 4) for a batch of up to 16,
// (4, 2, 2) above.
template <int MG, int kNT, int kUnroll>
__global__ __launch_bounds__(kOThreads) void oproj_kernel(const uint8_t* __restrict__ F,
                                                          const float* __restrict__ z,
                                                          float* __restrict__ out, int K,
                                                          int hidden, int batch) {
  __shared__ float s_red[kOWaves / 2][MG][kNT][4][kWave];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int kq = lane >> 4, col = lane & 15;
  const int ntiles = hidden / 16;
  const int t0 = blockIdx.x * kNT;
  const int ksteps = (K + 31) / 32;
  const uint8_t* Frow[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    const int tile = min(t0 + t, ntiles - 1);  // past the last tile: read it, store nothing
    Frow[t] = F + static_cast<size_t>(tile * 16 + col) * K * 2;
  }
  const int mtiles = (batch + 15) / 16;
  for (int mg = 0; mg < mtiles; mg += MG) {
    const int mcount = min(MG, mtiles - mg);
    f32x4 acc[MG][kNT];
#pragma unroll
    for (int m = 0; m < MG; ++m)
#pragma unroll
      for (int t = 0; t < kNT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = wave; s0 < ksteps; s0 += kOWaves * kUnroll) {
      // loads of kUnroll steps first (steps past the end read step 0 with zero
      // weight fragments; rows past the batch read row 0 and are dropped)
      uint4 bf[kUnroll][kNT];
      float4 zf[kUnroll][MG][2];
      bool kv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int s = s0 + u * kOWaves;
        int ci = s * 32 + kq * 8;
        kv[u] = (s < ksteps) && ci < K;
        if (!kv[u]) ci = 0;
#pragma unroll
        for (int t = 0; t < kNT; ++t) bf[u][t] = load16(Frow[t] + static_cast<size_t>(ci) * 2);
#pragma unroll
        for (int m = 0; m < MG; ++m) {
          int row = (mg + m) * 16 + col;
          if (m >= mcount || row >= batch) row = 0;
          const float* zr = z + static_cast<size_t>(row) * K + ci;
          zf[u][m][0] = *reinterpret_cast<const float4*>(zr);
          zf[u][m][1] = *reinterpret_cast<const float4*>(zr + 4);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
        for (int m = 0; m < MG; ++m) {
          const float x[8] = {zf[u][m][0].x, zf[u][m][0].y, zf[u][m][0].z, zf[u][m][0].w,
                              zf[u][m][1].x, zf[u][m][1].y, zf[u][m][1].z, zf[u][m][1].w};
          bf16x8 hi, lo;
          split_bf16x8(x, hi, lo);
#pragma unroll
          for (int t = 0; t < kNT; ++t) {
            const bf16x8 b = kv[u] ? __builtin_bit_cast(bf16x8, bf[u][t])
                                   : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
            acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, b, acc[m][t], 0, 0, 0);
            acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, b, acc[m][t], 0, 0, 0);
          }
        }
      }
    }
    // the waves' partial tiles are summed through LDS in a fixed order (the
    // same every run): waves w and w + 4 pair up, then the four pair sums are
    // added in order; lane holds batch rows 4*kq + v of output column col
    constexpr int kHalf = kOWaves / 2;
    if (wave >= kHalf) {
#pragma unroll
      for (int m = 0; m < MG; ++m)
#pragma unroll
        for (int t = 0; t < kNT; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v) s_red[wave - kHalf][m][t][v][lane] = acc[m][t][v];
    }
    __syncthreads();
    if (wave < kHalf) {
#pragma unroll
      for (int m = 0; m < MG; ++m)
#pragma unroll
        for (int t = 0; t < kNT; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v) s_red[wave][m][t][v][lane] += acc[m][t][v];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < MG * kNT * 4 * kWave; i += kOThreads) {
      const int m = i / (kNT * 4 * kWave), t = (i / (4 * kWave)) % kNT, v = (i / kWave) % 4;
      const int l = i % kWave;
      const int row = (mg + m) * 16 + 4 * (l >> 4) + v;
      if (m >= mcount || row >= batch || t0 + t >= ntiles) continue;
      float sum = s_red[0][m][t][v][l];
#pragma unroll
      for (int w = 1; w < kHalf; ++w) sum += s_red[w][m][t][v][l];
      out[static_cast<size_t>(row) * hidden + (t0 + t) * 16 + (l & 15)] = sum;
    }
    __syncthreads();
  }
}

template <int D>
hipError_t fold_by_rv(const FoldArgs& a, hipStream_t s) {
  dim3 grid(a.hidden / 16, a.dm.Hq);
  switch (a.dm.RV) {
#define KVLR_FOLD_CASE(R)                                                                         \
  case R:                                                                                         \
    hipLaunchKernelGGL((fold_kernel<D, R>), grid, dim3(kWave), 0, s,                              \
                       static_cast<const uint8_t*>(a.W_o), static_cast<const uint8_t*>(a.B_v),   \
                       static_cast<uint16_t*>(a.F), a.dm.Hq, a.dm.G);                            \
    return hipGetLastError();
    KVLR_FOLD_CASE(16)
    KVLR_FOLD_CASE(32)
    KVLR_FOLD_CASE(64)
#undef KVLR_FOLD_CASE
    case 128:
      if constexpr (D == 128) {
        hipLaunchKernelGGL((fold_kernel<D, 128>), grid, dim3(kWave), 0, s,
                           static_cast<const uint8_t*>(a.W_o), static_cast<const uint8_t*>(a.B_v),
                           static_cast<uint16_t*>(a.F), a.dm.Hq, a.dm.G);
        return hipGetLastError();
      }
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fold(const FoldArgs& a, hipStream_t s) {
  if (a.dm.D == 64) return fold_by_rv<64>(a, s);
  if (a.dm.D == 128) return fold_by_rv<128>(a, s);
  return hipErrorInvalidValue;
}

// (MG, kNT, kUnroll) for a batch of up to 16 and above
#ifndef KVLR_OPROJ_S_UNROLL
#define KVLR_OPROJ_S_UNROLL 4
#endif
#ifndef KVLR_OPROJ_L_MG
#define KVLR_OPROJ_L_MG 4
#endif
#ifndef KVLR_OPROJ_L_NT
#define KVLR_OPROJ_L_NT 2
#endif
#ifndef KVLR_OPROJ_L_UNROLL
#define KVLR_OPROJ_L_UNROLL 2
#endif

hipError_t launch_oproj(const OprojArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const int K = a.dm.Hq * a.dm.RV;
  const int ntiles = a.hidden / 16;
  if (a.batch <= 16)
    hipLaunchKernelGGL((oproj_kernel<1, 1, KVLR_OPROJ_S_UNROLL>), dim3(ntiles), dim3(kOThreads), 0, s,
                       static_cast<const uint8_t*>(a.F), a.z, a.out, K, a.hidden, a.batch);
  else
    hipLaunchKernelGGL((oproj_kernel<KVLR_OPROJ_L_MG, KVLR_OPROJ_L_NT, KVLR_OPROJ_L_UNROLL>),
                       dim3((ntiles + KVLR_OPROJ_L_NT - 1) / KVLR_OPROJ_L_NT), dim3(kOThreads), 0, s,
                       static_cast<const uint8_t*>(a.F), a.z, a.out, K, a.hidden, a.batch);
  return hipGetLastError();
}

}  // namespace kvlr
