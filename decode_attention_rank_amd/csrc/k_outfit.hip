// Joint fit of the value decoders across attention partitions.
//
// BasisKV: Value Latents for Communication and Key Routing, English abstract:
// the low-rank factors are optimised jointly across the per-GPU attention
// partitions against the complete attention output, rather than each
// partition on its own; method details (key design): the loss couples every
// GPU's attention partition; key innovation: value compression is tied to
// the output projection.
//
// With the value encoders A_g fixed (the cache's latents exist before any
// query), head h's latent output is z_h = x_h A_{h/G} for its exact output
// x_h. The joint decoder of the complete output from every partition's
// latents is the least-squares fit
//   D = argmin sum_n |x_n - z_n D|^2 = (Z^T Z)^-1 Z^T X,
// X [n][H_q d] the outputs, Z [n][H_q r] the latents; folded through the
// output projection it gives F = W_o D^T, the least-squares map from latents
// to W_o x for every W_o.
//
// GPU work (all dense contractions on the float32 matrix cores,
// v_mfma_f32_16x16x4_f32, with float32 sums over runs of 256 and float64
// sums of the runs): Z = X A per head; the moments Z^T Z and Z^T X; the fold
// F = W_o D^T. The host solves the normal equations in float64
// (kvlr_host_solve.cpp).

#include <math.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "kvlr_device.h"
#include "kvlr_internal.h"

namespace kvlr {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;   // output tile edge per workgroup
constexpr int kKs = 16;     // reduction elements per LDS stage
constexpr int kRun = 256;   // reduction elements summed in float32 before float64

// Element loads and stores by storage type: float, double, or bf16 (raw bits).
struct Bf16Raw {};
template <class T> struct Elem;
template <> struct Elem<float> {
  __device__ static float get(const void* p, long i) { return static_cast<const float*>(p)[i]; }
  __device__ static void put(void* p, long i, double v, bool acc) {
    float* q = static_cast<float*>(p);
    q[i] = static_cast<float>(acc ? q[i] + v : v);
  }
};
template <> struct Elem<double> {
  __device__ static float get(const void* p, long i) {
    return static_cast<float>(static_cast<const double*>(p)[i]);
  }
  __device__ static void put(void* p, long i, double v, bool acc) {
    double* q = static_cast<double*>(p);
    q[i] = acc ? q[i] + v : v;
  }
};
template <> struct Elem<Bf16Raw> {
  __device__ static float get(const void* p, long i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  }
  __device__ static void put(void* p, long i, double v, bool) {
    static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(f32_to_bf16_rne(static_cast<float>(v)));
  }
};

// C(m, n) (+)= sum_k A(m, k) B(k, n) over batch z, with
//   A(m, k) = A[z*saz + m*sam + k*sak]
//   B(k, n) = B[(z / bdiv)*sbz + k*sbk + n*sbn]
//   C(m, n) = C[z*scz + m*scm + n*scn]
struct GemmArgs {
  int M, N, K;
  const void* A;
  long sam, sak, saz;
  const void* B;
  long sbk, sbn, sbz;
  int bdiv;
  void* C;
  long scm, scn, scz;
  int accumulate;
};

// One 64 x 64 tile of C per workgroup; wave w owns the 32 x 32 quarter
// (w / 2, w % 2) as 2 x 2 matrix-core tiles. Operands are staged through
// double-buffered LDS, 16 reduction elements per stage; the next stage's
// global loads are in flight while the current one is multiplied. Loads are
// laid out along whichever operand stride is 1, so they coalesce.
template <class TA, class TB, class TC>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g) {
  __shared__ float sA[2][kKs][kTile + 4];
  __shared__ float sB[2][kKs][kTile + 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.x * kTile, n0 = blockIdx.y * kTile;
  const long z = blockIdx.z;
  const long abase = z * g.saz, bbase = (z / g.bdiv) * g.sbz;
  const bool a_kfast = (g.sak == 1), b_nfast = (g.sbn == 1);

  float ra[4], rb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * kThreads;
      const int kk = a_kfast ? (e & 15) : (e >> 6);
      const int mm = a_kfast ? (e >> 4) : (e & 63);
      const int m = m0 + mm, k = k0 + kk;
      ra[i] = (m < g.M && k < g.K) ? Elem<TA>::get(g.A, abase + m * g.sam + k * g.sak) : 0.f;
      const int kb = b_nfast ? (e >> 6) : (e & 15);
      const int nn = b_nfast ? (e & 63) : (e >> 4);
      const int n = n0 + nn, kq = k0 + kb;
      rb[i] = (n < g.N && kq < g.K) ? Elem<TB>::get(g.B, bbase + kq * g.sbk + n * g.sbn) : 0.f;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * kThreads;
      const int kk = a_kfast ? (e & 15) : (e >> 6);
      const int mm = a_kfast ? (e >> 4) : (e & 63);
      sA[buf][kk][mm] = ra[i];
      const int kb = b_nfast ? (e >> 6) : (e & 15);
      const int nn = b_nfast ? (e & 63) : (e >> 4);
      sB[buf][kb][nn] = rb[i];
    }
  };

  const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;
  const int row = lane & 15, kq = lane >> 4;
  f32x4 acc[2][2];
  double acc64[2][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < 4; ++v) acc64[i][j][v] = 0.0;
    }
  auto flush = [&] {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc64[i][j][v] += static_cast<double>(acc[i][j][v]);
        acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
  };

  const int nst = (g.K + kKs - 1) / kKs;
  load(0);
  stash(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    if (st + 1 < nst) load((st + 1) * kKs);
#pragma unroll
    for (int s = 0; s < kKs / 4; ++s) {
      const int k = 4 * s + kq;
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = sA[cur][k][wr + 16 * i + row];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = sB[cur][k][wc + 16 * j + row];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (((st + 1) * kKs) % kRun == 0) flush();
    if (st + 1 < nst) stash(cur ^ 1);
    __syncthreads();
  }
  flush();
  // lane holds rows 4 * (lane / 16) + v of column lane % 16 of each tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wr + 16 * i + 4 * kq + v;
        const int n = n0 + wc + 16 * j + row;
        if (m < g.M && n < g.N)
          Elem<TC>::put(g.C, z * g.scz + m * g.scm + n * g.scn, acc64[i][j][v], g.accumulate != 0);
      }
}

template <class TA, class TB, class TC>
hipError_t gemm(const GemmArgs& g, int batch, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || batch <= 0) return hipSuccess;
  dim3 grid((g.M + kTile - 1) / kTile, (g.N + kTile - 1) / kTile, batch);
  hipLaunchKernelGGL((gemm_kernel<TA, TB, TC>), grid, dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_joint_moments(const JointArgs& a, hipStream_t s) {
  const int Hq = a.dm.Hq, D = a.dm.D, R = a.dm.RV, G = a.dm.G;
  const long nl = static_cast<long>(Hq) * R, nx = static_cast<long>(Hq) * D;
  if (a.n == 0) return hipSuccess;
  // Z[n][h r + j] = sum_i X[n][h][i] A_{h/G}[i][j], one batch entry per head
  GemmArgs z{};
  z.M = a.n;
  z.N = R;
  z.K = D;
  z.A = a.x;
  z.sam = nx;
  z.sak = 1;
  z.saz = D;
  z.B = a.A_v;
  z.sbk = R;
  z.sbn = 1;
  z.sbz = static_cast<long>(D) * R;
  z.bdiv = G;
  z.C = a.z;
  z.scm = nl;
  z.scn = 1;
  z.scz = R;
  hipError_t e = a.dm.dtype == 0 ? gemm<float, Bf16Raw, float>(z, Hq, s) : gemm<float, float, float>(z, Hq, s);
  if (e != hipSuccess) return e;
  // Z^T Z and Z^T X: reductions over the samples
  GemmArgs m{};
  m.M = static_cast<int>(nl);
  m.K = a.n;
  m.A = a.z;
  m.sam = 1;
  m.sak = nl;
  m.sbn = 1;
  m.bdiv = 1;
  m.scn = 1;
  m.accumulate = a.accumulate;
  m.N = static_cast<int>(nl);
  m.B = a.z;
  m.sbk = nl;
  m.C = a.zz;
  m.scm = nl;
  e = gemm<float, float, double>(m, 1, s);
  if (e != hipSuccess) return e;
  m.N = static_cast<int>(nx);
  m.B = a.x;
  m.sbk = nx;
  m.C = a.zx;
  m.scm = nx;
  return gemm<float, float, double>(m, 1, s);
}

hipError_t launch_joint_fold(const JointFoldArgs& a, hipStream_t s) {
  // F[h][j] = sum_k W_o[h][k] D[j][k]
  const long nl = static_cast<long>(a.dm.Hq) * a.dm.RV, nx = static_cast<long>(a.dm.Hq) * a.dm.D;
  GemmArgs f{};
  f.M = a.hidden;
  f.N = static_cast<int>(nl);
  f.K = static_cast<int>(nx);
  f.A = a.W_o;
  f.sam = nx;
  f.sak = 1;
  f.B = a.Dm;
  f.sbk = 1;
  f.sbn = nx;
  f.bdiv = 1;
  f.C = a.F;
  f.scm = nl;
  f.scn = 1;
  return gemm<Bf16Raw, float, Bf16Raw>(f, 1, s);
}

// Host: D = zz^-1 zx by Cholesky (zz = L L^T, row-major lower L), then the
// forward and back substitutions for every right-hand side column, columns
// spread over threads. Fails when a pivot falls to 1e-12 of the largest
// diagonal entry (latents that the samples do not determine).
}  // namespace kvlr
