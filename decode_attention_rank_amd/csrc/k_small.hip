// Query projection, up-projection and workspace fill.
//
// BasisKV: Value Latents for Communication and Key Routing, English abstract.
//  - Scoring against latents needs the query mapped through the same
//    factors: q_hat = q W_pred^T (what the value latent predicts of the key),
//    q_tilde = q B_k^T (residual or key latent).
//  - Value compression is tied to the output projection: the decoder B_v is
//    applied once per query head to z = sum_t p_t v_t. This is a small dense
//    contraction ([B*G x r_v] x [r_v x d] per KV head) and runs on the float32
//    matrix cores (v_mfma_f32_16x16x4_f32) with float32 accumulation.

#include "kvlr_device.h"
#include "kvlr_gemm_tile.h"
#include "kvlr_internal.h"

namespace kvlr {
namespace {


// q_proj rows: [q W_pred^T (exact mode only), q B_k^T]. Grid: (row tiles,
// output-column tiles, KV heads).
template <class S, int D>
__global__ __launch_bounds__(64) void qproj_kernel(const uint8_t* __restrict__ W_pred,
                                                   const uint8_t* __restrict__ B_k,
                                                   const float* __restrict__ q,
                                                   float* __restrict__ q_proj, int B, int Hq,
                                                   int Hkv, int G, int RV, int RK, int exact) {
  qproj_tile<S, D>(W_pred, B_k, q, q_proj, B, Hq, G, RV, RK, exact, blockIdx.x, blockIdx.y,
                   blockIdx.z);
}

// o = z B_v per KV group. Grid: (row tiles, D / 16, KV heads).
template <class S, int RV, int D>
__global__ __launch_bounds__(64) void upproject_kernel(const float* __restrict__ z,
                                                       const uint8_t* __restrict__ B_v,
                                                       float* __restrict__ o, int B, int Hq,
                                                       int Hkv, int G) {
  const int g = blockIdx.z;
  small_gemm_tile<S, RV, false>(z, RV, B_v + static_cast<size_t>(g) * RV * D * S::ELEM_BYTES, D,
                                B * G, blockIdx.x, blockIdx.y * 16, G, Hq, g, o, D, 0);
}

__global__ void zero_fill_kernel(uint4* __restrict__ p, size_t n16, uint8_t* __restrict__ tail,
                                 size_t ntail) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0)
    for (size_t i = threadIdx.x; i < ntail; i += blockDim.x) tail[i] = 0;
}

template <class S, int RV>
hipError_t up_by_d(const UpprojArgs& a, hipStream_t s) {
  dim3 grid((a.batch * a.dm.G + 15) / 16, a.dm.D / 16, a.dm.Hkv);
  switch (a.dm.D) {
    case 64:
      hipLaunchKernelGGL((upproject_kernel<S, RV, 64>), grid, dim3(64), 0, s, a.z,
                         static_cast<const uint8_t*>(a.B_v), a.o, a.batch, a.dm.Hq, a.dm.Hkv,
                         a.dm.G);
      return hipGetLastError();
    case 128:
      hipLaunchKernelGGL((upproject_kernel<S, RV, 128>), grid, dim3(64), 0, s, a.z,
                         static_cast<const uint8_t*>(a.B_v), a.o, a.batch, a.dm.Hq, a.dm.Hkv,
                         a.dm.G);
      return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

template <class S, int D>
hipError_t qproj_t(const QprojArgs& a, hipStream_t s) {
  const int width = (a.dm.exact ? a.dm.RV : 0) + a.dm.RK;
  dim3 grid((a.batch * a.dm.G + 15) / 16, width / 16, a.dm.Hkv);
  hipLaunchKernelGGL((qproj_kernel<S, D>), grid, dim3(64), 0, s,
                     static_cast<const uint8_t*>(a.W_pred), static_cast<const uint8_t*>(a.B_k),
                     a.q, a.q_proj, a.batch, a.dm.Hq, a.dm.Hkv, a.dm.G, a.dm.RV, a.dm.RK,
                     a.dm.exact);
  return hipGetLastError();
}

template <class S>
hipError_t qproj_by_d(const QprojArgs& a, hipStream_t s) {
  switch (a.dm.D) {
    case 64: return qproj_t<S, 64>(a, s);
    case 128: return qproj_t<S, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class S>
hipError_t up_by_rv(const UpprojArgs& a, hipStream_t s) {
  switch (a.dm.RV) {
    case 16: return up_by_d<S, 16>(a, s);
    case 32: return up_by_d<S, 32>(a, s);
    case 64: return up_by_d<S, 64>(a, s);
    case 128: return up_by_d<S, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

// Page tables against the cache: each sequence's length within its table
// row, and every entry that length uses within [0, num_phys). One workgroup
// per sequence; each wave adds its count of bad entries once.
__global__ __launch_bounds__(256) void check_tables_kernel(const int32_t* __restrict__ seq_lens,
                                                           const int32_t* __restrict__ page_table,
                                                           int max_pages, int P, int num_phys,
                                                           uint32_t* __restrict__ errors) {
  const int b = blockIdx.x;
  const int L = seq_lens[b];
  if (threadIdx.x == 0 && (L < 0 || L > max_pages * P)) atomicOr(&errors[0], 2u);
  const int n = (table_len(L, max_pages, P) + P - 1) / P;
  uint32_t bad = 0;
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    const int id = page_table[static_cast<size_t>(b) * max_pages + j];
    bad += (id < 0 || id >= num_phys) ? 1u : 0u;
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) bad += __shfl_xor(bad, off, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0 && bad) {
    atomicOr(&errors[0], 1u);
    atomicAdd(&errors[1], bad);
  }
}

}  // namespace

hipError_t launch_check_tables(const int32_t* seq_lens, const int32_t* page_table, int max_pages,
                               int P, int num_phys, int batch, uint32_t* errors, hipStream_t s) {
  hipError_t e = launch_zero_fill(errors, 2 * sizeof(uint32_t), s);
  if (e != hipSuccess || batch == 0) return e;
  hipLaunchKernelGGL(check_tables_kernel, dim3(batch), dim3(256), 0, s, seq_lens, page_table, max_pages, P,
                     num_phys, errors);
  return hipGetLastError();
}

hipError_t launch_qproj(const QprojArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  if (a.dm.dtype == 0) return qproj_by_d<BF16>(a, s);
  return qproj_by_d<F32>(a, s);
}

hipError_t launch_upproject(const UpprojArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  if (a.dm.dtype == 0) return up_by_rv<BF16>(a, s);
  return up_by_rv<F32>(a, s);
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  const size_t ntail = bytes - n16 * 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_fill_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<uint4*>(p), n16, static_cast<uint8_t*>(p) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace kvlr
