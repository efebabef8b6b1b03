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
#include "kvlr_internal.h"

namespace kvlr {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One workgroup per (sequence, KV head): the G query heads share the factor rows.
template <class S>
__global__ __launch_bounds__(256) void qproj_kernel(const uint8_t* __restrict__ W_pred,
                                                    const uint8_t* __restrict__ B_k,
                                                    const float* __restrict__ q,
                                                    float* __restrict__ q_proj, int Hq, int Hkv,
                                                    int G, int D, int RV, int RK, int exact) {
  extern __shared__ float s_q[];  // [G][D]
  constexpr int CH = S::CH;
  const int pair = blockIdx.x;
  const int b = pair / Hkv;
  const int g = pair - b * Hkv;
  const float* qg = q + static_cast<size_t>(b * Hq + g * G) * D;
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) s_q[i] = qg[i];
  __syncthreads();
  const int RVe = exact ? RV : 0;
  const int Wd = RVe + RK;
  for (int i = threadIdx.x; i < G * Wd; i += blockDim.x) {
    const int h = i / Wd, o = i - h * Wd;
    const uint8_t* row = (o < RVe)
        ? W_pred + (static_cast<size_t>(g) * RV + o) * D * S::ELEM_BYTES
        : B_k + (static_cast<size_t>(g) * RK + (o - RVe)) * D * S::ELEM_BYTES;
    const float* qh = s_q + h * D;
    float acc = 0.f;
    for (int c = 0; c < D / CH; ++c) {
      float x[CH];
      S::unpack(load16(row + c * 16), x);
#pragma unroll
      for (int e = 0; e < CH; ++e) acc = fmaf(qh[c * CH + e], x[e], acc);
    }
    q_proj[(static_cast<size_t>(b) * Hq + g * G + h) * Wd + o] = acc;
  }
}

// One wave per 16 (sequence, head) rows of one KV group, all d columns.
template <class S, int RV, int D>
__global__ __launch_bounds__(64) void upproject_kernel(const float* __restrict__ z,
                                                       const uint8_t* __restrict__ B_v,
                                                       float* __restrict__ o, int B, int Hq,
                                                       int Hkv, int G) {
  constexpr int NT = D / 16;
  const int g = blockIdx.y;
  const int lane = threadIdx.x;
  const int rows = B * G;
  // A operand row of this lane: l % 16; k offset: l / 16
  const int ra = blockIdx.x * 16 + (lane & 15);
  const bool va = ra < rows;
  const int ba = va ? ra / G : 0;
  const int ha = va ? g * G + (ra - ba * G) : 0;
  const float* zr = z + (static_cast<size_t>(ba) * Hq + ha) * RV;
  const int kq = lane >> 4;
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const size_t bbase = static_cast<size_t>(g) * RV * D;
#pragma unroll 4
  for (int k0 = 0; k0 < RV; k0 += 4) {
    const float a = va ? zr[k0 + kq] : 0.f;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const float bv = S::load1(B_v, bbase + static_cast<size_t>(k0 + kq) * D + n * 16 + (lane & 15));
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, acc[n], 0, 0, 0);
    }
  }
  // D layout: lane holds rows 4*(l/16)+i, column l%16 of each 16x16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = blockIdx.x * 16 + 4 * (lane >> 4) + i;
    if (r >= rows) continue;
    const int bb = r / G;
    const int hh = g * G + (r - bb * G);
    float* orow = o + (static_cast<size_t>(bb) * Hq + hh) * D;
#pragma unroll
    for (int n = 0; n < NT; ++n) orow[n * 16 + (lane & 15)] = acc[n][i];
  }
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
  dim3 grid((a.batch * a.dm.G + 15) / 16, a.dm.Hkv);
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

template <class S>
hipError_t up_by_rv(const UpprojArgs& a, hipStream_t s) {
  switch (a.dm.RV) {
    case 16: return up_by_d<S, 16>(a, s);
    case 32: return up_by_d<S, 32>(a, s);
    case 64: return up_by_d<S, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_qproj(const QprojArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const size_t lds = static_cast<size_t>(a.dm.G) * a.dm.D * sizeof(float);
  dim3 grid(a.batch * a.dm.Hkv);
  if (a.dm.dtype == 0)
    hipLaunchKernelGGL((qproj_kernel<BF16>), grid, dim3(256), lds, s,
                       static_cast<const uint8_t*>(a.W_pred), static_cast<const uint8_t*>(a.B_k),
                       a.q, a.q_proj, a.dm.Hq, a.dm.Hkv, a.dm.G, a.dm.D, a.dm.RV, a.dm.RK,
                       a.dm.exact);
  else
    hipLaunchKernelGGL((qproj_kernel<F32>), grid, dim3(256), lds, s,
                       static_cast<const uint8_t*>(a.W_pred), static_cast<const uint8_t*>(a.B_k),
                       a.q, a.q_proj, a.dm.Hq, a.dm.Hkv, a.dm.G, a.dm.D, a.dm.RV, a.dm.RK,
                       a.dm.exact);
  return hipGetLastError();
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
