// Factor fitting from sample keys and values (a calibration-time step).
//
// BasisKV: Value Latents for Communication and Key Routing, English abstract
// (low-rank K/V projections; the value latent predicts part of the key and a
// key-specific residual holds what the value cannot recover) and method
// details (key design: the choice of the low-rank factors). The pages do not
// spell out the fit; this is the staged reading, per KV head:
//   A_v    = top-r_v eigenvectors of V^T V,                  B_v = A_v^T
//   W_pred = (v^T v)^-1 v^T K with v = V A_v                 (least squares)
//   A_k    = top-r_k eigenvectors of R^T R, R = K - v W_pred (exact keys)
//            or of K^T K                                      (latent keys)
//   B_k    = A_k^T
// Everything follows from three second moments, C_VV = V^T V, C_KK = K^T K
// and C_VK = V^T K, because with P = A_v^T C_VK = v^T K and
// M = A_v^T C_VV A_v = v^T v:  W_pred = M^-1 P  and  R^T R = C_KK - P^T W_pred.
//
//  - moments_mfma_kernel (bf16 samples): a workgroup takes a run of tokens of
//    one KV head and forms the upper block triangle of Z^T Z, Z = [V K]
//    (V^T V, K^T K, V^T K) on the matrix cores: v_mfma_f32_16x16x32_bf16,
//    exact bf16 products, float32 sums. Tokens are staged 128 at a time into
//    double-buffered LDS directly in fragment order (8 tokens of one
//    dimension per lane), so an operand is one 16-byte LDS read; each wave
//    owns a 4x4-block patch of the triangle and reuses every fragment it
//    reads in 4 or 5 products. The next stage's loads are in flight while
//    the current one is multiplied.
//  - moments_valu_kernel (f32 samples): the same partial sums on the vector
//    ALUs, one 8x8 (or 4x4) block of one moment per thread.
//  - moments_sum_kernel adds the per-run partials in a fixed order into
//    float64 moments (optionally onto what the buffer already holds) and
//    mirrors the symmetric moments' lower triangle.
//  - The host solves the small symmetric eigenproblems in float64:
//    Householder reduction to tridiagonal form, then implicit QR steps with
//    the Wilkinson shift (Golub and Van Loan, Matrix Computations, the
//    symmetric QR algorithm), eigenvectors accumulated throughout.

#include <algorithm>
#include <cmath>
#include <thread>
#include <vector>

#include "kvlr_device.h"
#include "kvlr_internal.h"

namespace kvlr {
namespace {

constexpr int kStageTok = 128;   // tokens staged per LDS fill (double-buffered: 128 KB)
constexpr int kFitGrid = 256;    // workgroups over all heads: one per compute unit

template <int D>
struct MomLayout {
  static constexpr int NB = D / 16;                    // 16-dimension blocks per tensor
  static constexpr int WAVES = NB;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int KSTEPS = kStageTok / 32;        // 32-token matrix-core k-steps
  static constexpr int FRAG_DW = kWave * 4;            // one fragment: 64 lanes x 16 bytes
  static constexpr int RB_DW = KSTEPS * FRAG_DW + 4;   // +16 bytes: blocks start on rotating banks
  static constexpr int BUF_DW = 2 * NB * RB_DW;        // V blocks then K blocks
  static constexpr int CHUNKS = D / 8;                 // 16-byte chunks per token row
  static constexpr int TASKS = 2 * (kStageTok / 4) * CHUNKS / THREADS;  // staging tasks per thread
  static_assert(TASKS * THREADS == 2 * (kStageTok / 4) * CHUNKS, "staging tasks divide evenly");
};

// The moments are the blocks of Z^T Z, Z = [V K] (2 NB blocks of 16
// dimensions): V^T V, K^T K and V^T K. Only the upper triangle (block row <=
// block column) is formed; the sum kernel mirrors the rest. A wave owns a
// patch of 4x4 blocks (diagonal patches are triangles, two per wave), so it
// reads 8 fragments per k-step and reuses each in 4 or 5 products.
struct WaveJob {
  int nf, nt;
  int f[8];            // Z blocks whose fragments the wave reads
  int a[20], b[20];    // tile t = fragment f[a[t]]^T times fragment f[b[t]]
};

template <int D>
constexpr WaveJob wave_job(int w) {
  WaveJob j{};
  if (D == 128) {
    const int offI[6] = {0, 0, 0, 1, 1, 2}, offJ[6] = {1, 2, 3, 2, 3, 3};
    if (w < 6) {  // an off-diagonal 4x4 patch: 16 tiles
      j.nf = 8;
      for (int r = 0; r < 4; ++r) {
        j.f[r] = 4 * offI[w] + r;
        j.f[4 + r] = 4 * offJ[w] + r;
      }
      for (int r = 0; r < 4; ++r)
        for (int c = 0; c < 4; ++c) {
          j.a[j.nt] = r;
          j.b[j.nt] = 4 + c;
          ++j.nt;
        }
    } else {  // two diagonal patches, upper triangles: 2 x 10 tiles
      const int p0 = 2 * (w - 6);
      j.nf = 8;
      for (int r = 0; r < 4; ++r) {
        j.f[r] = 4 * p0 + r;
        j.f[4 + r] = 4 * (p0 + 1) + r;
      }
      for (int h = 0; h < 2; ++h)
        for (int r = 0; r < 4; ++r)
          for (int c = r; c < 4; ++c) {
            j.a[j.nt] = 4 * h + r;
            j.b[j.nt] = 4 * h + c;
            ++j.nt;
          }
    }
  } else {  // D == 64: Z has 8 blocks, 36 upper tiles over 4 waves
    if (w < 2) {  // half of the V^T K patch: block rows 2w, 2w+1
      j.nf = 6;
      j.f[0] = 2 * w;
      j.f[1] = 2 * w + 1;
      for (int c = 0; c < 4; ++c) j.f[2 + c] = 4 + c;
      for (int r = 0; r < 2; ++r)
        for (int c = 0; c < 4; ++c) {
          j.a[j.nt] = r;
          j.b[j.nt] = 2 + c;
          ++j.nt;
        }
    } else {  // V^T V (w = 2) or K^T K (w = 3) upper triangle
      j.nf = 4;
      for (int r = 0; r < 4; ++r) j.f[r] = 4 * (w - 2) + r;
      for (int r = 0; r < 4; ++r)
        for (int c = r; c < 4; ++c) {
          j.a[j.nt] = r;
          j.b[j.nt] = c;
          ++j.nt;
        }
    }
  }
  return j;
}

// bf16 half e (0..7) of a 16-byte chunk
__device__ __forceinline__ uint32_t half_of(const uint4& x, int e) {
  const uint32_t w = e < 2 ? x.x : (e < 4 ? x.y : (e < 6 ? x.z : x.w));
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// The whole run for wave W of the workgroup (all waves pass the same
// barriers; only the products differ).
template <int D, int W>
__device__ __forceinline__ void moments_run(const uint8_t* __restrict__ k,
                                            const uint8_t* __restrict__ v,
                                            float* __restrict__ partial, int n, int Hkv,
                                            int chunk_tokens, uint32_t* lds) {
  using L = MomLayout<D>;
  constexpr WaveJob J = wave_job<D>(W);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int c = blockIdx.x, g = blockIdx.y;
  const int t0 = c * chunk_tokens;
  const int t1 = min(t0 + chunk_tokens, n);
  const size_t row_bytes = static_cast<size_t>(Hkv) * D * 2;

  // staging task i of this thread: tensor i, 4-token group tg, 16-byte chunk ch
  const int ch = tid % L::CHUNKS;
  const int tg = (tid / L::CHUNKS) % (kStageTok / 4);
  const uint8_t* src[L::TASKS];
  int slot[L::TASKS];
#pragma unroll
  for (int i = 0; i < L::TASKS; ++i) {
    const int q = tid + i * L::THREADS;
    const int tt = q / ((kStageTok / 4) * L::CHUNKS);
    src[i] = (tt == 0 ? v : k) + static_cast<size_t>(g) * D * 2 + ch * 16;
    // (token 4 tg + u, dimension 8 ch + e) -> block ch/2 of tensor tt,
    // k-step tg/8, lane ((tg%8)/2)*16 + (ch%2)*8 + e, tokens 4 (tg%2) .. +3
    slot[i] = (tt * L::NB + ch / 2) * L::RB_DW + (tg / 8) * L::FRAG_DW +
              (((tg % 8) / 2) * 16 + (ch % 2) * 8) * 4 + 2 * (tg % 2);
  }
  // The next stage's tokens are loaded while the current one is multiplied.
  // Loads past the run's end read its last token and are zeroed, so every
  // load is unconditional.
  uint4 xa[L::TASKS][4];
  auto load_stage = [&](uint4 (&x)[L::TASKS][4], int base) {
#pragma unroll
    for (int i = 0; i < L::TASKS; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = base + 4 * tg + u;
        x[i][u] = load16(src[i] + static_cast<size_t>(min(t, t1 - 1)) * row_bytes);
        if (t >= t1) x[i][u] = make_uint4(0, 0, 0, 0);
      }
  };
  auto store_stage = [&](const uint4 (&x)[L::TASKS][4], uint32_t* buf) {
#pragma unroll
    for (int i = 0; i < L::TASKS; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint2 pk;
        pk.x = half_of(x[i][0], e) | (half_of(x[i][1], e) << 16);
        pk.y = half_of(x[i][2], e) | (half_of(x[i][3], e) << 16);
        *reinterpret_cast<uint2*>(&buf[slot[i] + e * 4]) = pk;
      }
  };

  f32x4 acc[J.nt];
#pragma unroll
  for (int t = 0; t < J.nt; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto multiply = [&](const uint32_t* cur) {
#pragma unroll
    for (int ks = 0; ks < L::KSTEPS; ++ks) {
      bf16x8 fr[J.nf];
#pragma unroll
      for (int i = 0; i < J.nf; ++i)
        fr[i] = *reinterpret_cast<const bf16x8*>(&cur[J.f[i] * L::RB_DW + ks * L::FRAG_DW + lane * 4]);
#pragma unroll
      for (int t = 0; t < J.nt; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[J.a[t]], fr[J.b[t]], acc[t], 0, 0, 0);
    }
  };

  uint32_t* buf0 = lds;
  uint32_t* buf1 = lds + L::BUF_DW;
  const int stages = (t1 - t0 + kStageTok - 1) / kStageTok;
  load_stage(xa, t0);
  store_stage(xa, buf0);
  __syncthreads();
  for (int s = 0; s < stages; ++s) {
    load_stage(xa, t0 + (s + 1) * kStageTok);
    multiply((s & 1) ? buf1 : buf0);
    store_stage(xa, (s & 1) ? buf0 : buf1);
    __syncthreads();  // next stage visible; this stage's buffer free for reuse
  }
  // lane holds rows 4*(lane/16) + r of column lane%16 of each 16x16 tile
  const int kq = lane >> 4, col = lane & 15;
#pragma unroll
  for (int t = 0; t < J.nt; ++t) {
    const int za = J.f[J.a[t]], zb = J.f[J.b[t]];
    const int m = zb < L::NB ? 0 : (za >= L::NB ? 1 : 2);
    const int row0 = (za % L::NB) * 16, col0 = (zb % L::NB) * 16;
    float* out = partial + ((static_cast<size_t>(c) * Hkv + g) * 3 + m) * D * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      out[static_cast<size_t>(row0 + 4 * kq + r) * D + col0 + col] = acc[t][r];
  }
}

template <int D>
__global__ __launch_bounds__(MomLayout<D>::THREADS) void moments_mfma_kernel(
    const uint8_t* __restrict__ k, const uint8_t* __restrict__ v, float* __restrict__ partial,
    int n, int Hkv, int chunk_tokens) {
  __shared__ __align__(16) uint32_t lds[2 * MomLayout<D>::BUF_DW];
  switch (threadIdx.x / kWave) {
#define KVLR_MOM_WAVE(W)                                                  \
  case W:                                                                 \
    if constexpr (W < MomLayout<D>::WAVES)                                \
      moments_run<D, W>(k, v, partial, n, Hkv, chunk_tokens, lds);        \
    break;
    KVLR_MOM_WAVE(0)
    KVLR_MOM_WAVE(1)
    KVLR_MOM_WAVE(2)
    KVLR_MOM_WAVE(3)
    KVLR_MOM_WAVE(4)
    KVLR_MOM_WAVE(5)
    KVLR_MOM_WAVE(6)
    KVLR_MOM_WAVE(7)
#undef KVLR_MOM_WAVE
  }
}

constexpr int kValuThreads = 256;
constexpr int kValuStage = 32;

// grid (run, moment, KV head); thread t owns a BS x BS block of the d x d
// moment (BS = d / 16). Moment 0: V^T V, 1: K^T K, 2: V^T K.
template <int D>
__global__ __launch_bounds__(kValuThreads) void moments_valu_kernel(
    const float* __restrict__ k, const float* __restrict__ v, float* __restrict__ partial, int n,
    int Hkv, int chunk_tokens) {
  constexpr int BS = D / 16;
  __shared__ float sx[kValuStage][D];
  __shared__ float sy[kValuStage][D];
  const int c = blockIdx.x, mom = blockIdx.y, g = blockIdx.z;
  const int tid = threadIdx.x;
  const int bi = tid / 16, bj = tid % 16;
  const float* X = (mom == 1) ? k : v;
  const float* Y = (mom == 0) ? v : k;
  const int t0 = c * chunk_tokens;
  const int t1 = min(t0 + chunk_tokens, n);
  float acc[BS][BS];
#pragma unroll
  for (int i = 0; i < BS; ++i)
#pragma unroll
    for (int j = 0; j < BS; ++j) acc[i][j] = 0.f;
  for (int ts = t0; ts < t1; ts += kValuStage) {
    for (int idx = tid; idx < kValuStage * (D / 4); idx += kValuThreads) {
      const int r = idx / (D / 4), cc = idx % (D / 4);
      const int t = ts + r;
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
      if (t < t1) {
        const size_t off = (static_cast<size_t>(t) * Hkv + g) * D + cc * 4;
        a = *reinterpret_cast<const float4*>(X + off);
        b = *reinterpret_cast<const float4*>(Y + off);
      }
      *reinterpret_cast<float4*>(&sx[r][cc * 4]) = a;
      *reinterpret_cast<float4*>(&sy[r][cc * 4]) = b;
    }
    __syncthreads();
    for (int r = 0; r < kValuStage; ++r) {
      float xi[BS], yj[BS];
#pragma unroll
      for (int i = 0; i < BS; ++i) {
        xi[i] = sx[r][bi * BS + i];
        yj[i] = sy[r][bj * BS + i];
      }
#pragma unroll
      for (int i = 0; i < BS; ++i)
#pragma unroll
        for (int j = 0; j < BS; ++j) acc[i][j] = fmaf(xi[i], yj[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* out = partial + ((static_cast<size_t>(c) * Hkv + g) * 3 + mom) * D * D;
#pragma unroll
  for (int i = 0; i < BS; ++i)
#pragma unroll
    for (int j = 0; j < BS; ++j) out[static_cast<size_t>(bi * BS + i) * D + bj * BS + j] = acc[i][j];
}

// Adds the per-run partials in run order. The symmetric moments (V^T V,
// K^T K) were formed only for block row <= block column: those sums are
// also written to the mirrored position.
__global__ __launch_bounds__(256) void moments_sum_kernel(const float* __restrict__ partial,
                                                          double* __restrict__ moments, int runs,
                                                          int D, size_t per_run, int accumulate) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= per_run) return;
  const int col = static_cast<int>(i % D), row = static_cast<int>((i / D) % D);
  const int m = static_cast<int>((i / (static_cast<size_t>(D) * D)) % 3);
  const bool sym = m < 2;
  if (sym && row / 16 > col / 16) return;
  double s = 0.0;
  int c = 0;
  for (; c + 8 <= runs; c += 8) {  // eight loads in flight, summed in run order
    float p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) p[u] = partial[static_cast<size_t>(c + u) * per_run + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += static_cast<double>(p[u]);
  }
  for (; c < runs; ++c) s += static_cast<double>(partial[static_cast<size_t>(c) * per_run + i]);
  moments[i] = (accumulate ? moments[i] : 0.0) + s;
  if (sym && row / 16 < col / 16) {
    const size_t mi = i - (static_cast<size_t>(row) * D + col) + static_cast<size_t>(col) * D + row;
    moments[mi] = (accumulate ? moments[mi] : 0.0) + s;
  }
}

// ---------------------------------------------------------------- host side

constexpr double kEps = 2.220446049250313e-16;

// Symmetric eigen-decomposition of the n x n row-major A (destroyed).
// On return lam[i] are the eigenvalues and row i of Zt (n x n) the unit
// eigenvector of lam[i]. Returns false if the QR steps did not converge.
bool sym_eig(std::vector<double>& A, int n, std::vector<double>& lam, std::vector<double>& Zt) {
  auto at = [&](int i, int j) -> double& { return A[static_cast<size_t>(i) * n + j]; };
  Zt.assign(static_cast<size_t>(n) * n, 0.0);
  for (int i = 0; i < n; ++i) Zt[static_cast<size_t>(i) * n + i] = 1.0;
  std::vector<double> hv(n), p(n), w(n), u(n);
  // Householder reduction: step j zeroes column j below the subdiagonal.
  for (int j = 0; j + 2 < n; ++j) {
    const int m = n - j - 1;
    double tail = 0.0;
    for (int i = 1; i < m; ++i) tail += at(j + 1 + i, j) * at(j + 1 + i, j);
    if (tail == 0.0) continue;
    const double x0 = at(j + 1, j);
    const double xn = std::sqrt(tail + x0 * x0);
    const double alpha = x0 > 0 ? -xn : xn;  // v0 = x0 - alpha adds magnitudes
    for (int i = 0; i < m; ++i) hv[i] = at(j + 1 + i, j);
    hv[0] = x0 - alpha;
    const double beta = 2.0 / (tail + hv[0] * hv[0]);
    // trailing block S <- H S H with H = I - beta hv hv^T
    double pv = 0.0;
    for (int i = 0; i < m; ++i) {
      double s = 0.0;
      for (int l = 0; l < m; ++l) s += at(j + 1 + i, j + 1 + l) * hv[l];
      p[i] = beta * s;
      pv += p[i] * hv[i];
    }
    const double kk = 0.5 * beta * pv;
    for (int i = 0; i < m; ++i) w[i] = p[i] - kk * hv[i];
    for (int i = 0; i < m; ++i)
      for (int l = 0; l < m; ++l) at(j + 1 + i, j + 1 + l) -= hv[i] * w[l] + w[i] * hv[l];
    at(j + 1, j) = at(j, j + 1) = alpha;
    for (int i = 1; i < m; ++i) at(j + 1 + i, j) = at(j, j + 1 + i) = 0.0;
    // accumulate: rows j+1.. of Zt <- H rows
    std::fill(u.begin(), u.end(), 0.0);
    for (int i = 0; i < m; ++i) {
      const double* zr = &Zt[static_cast<size_t>(j + 1 + i) * n];
      for (int l = 0; l < n; ++l) u[l] += hv[i] * zr[l];
    }
    for (int i = 0; i < m; ++i) {
      double* zr = &Zt[static_cast<size_t>(j + 1 + i) * n];
      const double f = beta * hv[i];
      for (int l = 0; l < n; ++l) zr[l] -= f * u[l];
    }
  }
  std::vector<double> a(n), b(std::max(n - 1, 1), 0.0);
  double anorm = 0.0;
  for (int i = 0; i < n; ++i) {
    a[i] = at(i, i);
    anorm = std::max(anorm, std::fabs(a[i]));
    if (i + 1 < n) {
      b[i] = at(i + 1, i);
      anorm = std::max(anorm, std::fabs(b[i]));
    }
  }
  auto negligible = [&](int i) {  // b[i] couples i and i + 1
    return std::fabs(b[i]) <= kEps * (std::fabs(a[i]) + std::fabs(a[i + 1])) ||
           std::fabs(b[i]) <= kEps * anorm;
  };
  auto rotate_rows = [&](int r0, double cs, double sn) {
    double* z0 = &Zt[static_cast<size_t>(r0) * n];
    double* z1 = z0 + n;
    for (int l = 0; l < n; ++l) {
      const double x = z0[l], y = z1[l];
      z0[l] = cs * x + sn * y;
      z1[l] = -sn * x + cs * y;
    }
  };
  int hi = n - 1;
  long steps = 0;
  while (hi > 0) {
    if (negligible(hi - 1)) {
      b[hi - 1] = 0.0;
      --hi;
      continue;
    }
    int lo = hi - 1;
    while (lo > 0 && !negligible(lo - 1)) --lo;
    if (lo > 0) b[lo - 1] = 0.0;
    if (++steps > 64L * n) return false;
    // one implicit QR step on the unreduced block lo..hi
    const double del = 0.5 * (a[hi - 1] - a[hi]);
    const double bb = b[hi - 1];
    const double mu = a[hi] - bb * bb / (del + std::copysign(std::hypot(del, bb), del));
    double x = a[lo] - mu, z = b[lo];
    for (int kk = lo; kk < hi; ++kk) {
      const double r = std::hypot(x, z);
      const double cs = r == 0.0 ? 1.0 : x / r, sn = r == 0.0 ? 0.0 : z / r;
      if (kk > lo) b[kk - 1] = r;
      const double ak = a[kk], ak1 = a[kk + 1], bk = b[kk];
      a[kk] = cs * cs * ak + 2.0 * cs * sn * bk + sn * sn * ak1;
      a[kk + 1] = sn * sn * ak - 2.0 * cs * sn * bk + cs * cs * ak1;
      b[kk] = cs * sn * (ak1 - ak) + (cs * cs - sn * sn) * bk;
      if (kk + 1 < hi) {
        z = sn * b[kk + 1];  // the bulge below the subdiagonal
        b[kk + 1] *= cs;
        x = b[kk];
      }
      rotate_rows(kk, cs, sn);
    }
  }
  lam = a;
  return true;
}

// Columns of out [n][r]: eigenvectors of the r largest eigenvalues, largest
// first (equal ones in index order), each with its largest-magnitude entry
// positive. lam_out [r] (may be null).
bool top_eigvecs(std::vector<double> C, int n, int r, double* out, double* lam_out) {
  std::vector<double> lam, Zt;
  if (!sym_eig(C, n, lam, Zt)) return false;
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return lam[x] > lam[y]; });
  for (int c = 0; c < r; ++c) {
    const double* z = &Zt[static_cast<size_t>(order[c]) * n];
    int big = 0;
    for (int i = 1; i < n; ++i)
      if (std::fabs(z[i]) > std::fabs(z[big])) big = i;
    const double sg = z[big] < 0 ? -1.0 : 1.0;
    for (int i = 0; i < n; ++i) out[static_cast<size_t>(i) * r + c] = sg * z[i];
    if (lam_out) lam_out[c] = lam[order[c]];
  }
  return true;
}

// Solves M X = Pm for the symmetric positive definite r x r M (Cholesky);
// Pm is r x m, overwritten with X. False if M is not (numerically) positive
// definite: a pivot at or below kPivotFloor of M's largest diagonal entry.
// M = v^T v has the chosen eigenvalues of V^T V on its diagonal, so this
// rejects latent directions with under a millionth of the leading
// direction's energy, below what float32-accumulated moments resolve.
constexpr double kPivotFloor = 1e-6;
bool spd_solve(std::vector<double> M, int r, std::vector<double>& Pm, int m) {
  auto at = [&](int i, int j) -> double& { return M[static_cast<size_t>(i) * r + j]; };
  double dmax = 0.0;
  for (int i = 0; i < r; ++i) dmax = std::max(dmax, at(i, i));
  if (!(dmax > 0.0)) return false;
  for (int j = 0; j < r; ++j) {
    double d = at(j, j);
    for (int l = 0; l < j; ++l) d -= at(j, l) * at(j, l);
    if (!(d > kPivotFloor * dmax)) return false;
    d = std::sqrt(d);
    at(j, j) = d;
    for (int i = j + 1; i < r; ++i) {
      double s = at(i, j);
      for (int l = 0; l < j; ++l) s -= at(i, l) * at(j, l);
      at(i, j) = s / d;
    }
  }
  for (int col = 0; col < m; ++col) {
    for (int i = 0; i < r; ++i) {  // L y = p
      double s = Pm[static_cast<size_t>(i) * m + col];
      for (int l = 0; l < i; ++l) s -= at(i, l) * Pm[static_cast<size_t>(l) * m + col];
      Pm[static_cast<size_t>(i) * m + col] = s / at(i, i);
    }
    for (int i = r - 1; i >= 0; --i) {  // L^T x = y
      double s = Pm[static_cast<size_t>(i) * m + col];
      for (int l = i + 1; l < r; ++l) s -= at(l, i) * Pm[static_cast<size_t>(l) * m + col];
      Pm[static_cast<size_t>(i) * m + col] = s / at(i, i);
    }
  }
  return true;
}

std::vector<double> symmetric_copy(const double* C, int D) {
  std::vector<double> S(C, C + static_cast<size_t>(D) * D);
  for (int i = 0; i < D; ++i)
    for (int j = i + 1; j < D; ++j) {
      const double m = 0.5 * (S[static_cast<size_t>(i) * D + j] + S[static_cast<size_t>(j) * D + i]);
      S[static_cast<size_t>(i) * D + j] = S[static_cast<size_t>(j) * D + i] = m;
    }
  return S;
}

// One KV head. mom: C_VV, C_KK, C_VK (each D x D). Outputs as in fit_solve.
FitStatus solve_head(const Dims& dm, const double* mom, double* A_v, double* A_k, double* W,
                     double* lam_v, double* lam_k) {
  const int D = dm.D, RV = dm.RV, RK = dm.RK;
  const size_t dd = static_cast<size_t>(D) * D;
  const double* Cvv = mom;
  const double* Ckk = mom + dd;
  const double* Cvk = mom + 2 * dd;
  if (!top_eigvecs(symmetric_copy(Cvv, D), D, RV, A_v, lam_v)) return FitStatus::kNoConvergence;
  if (!dm.exact) {
    if (!top_eigvecs(symmetric_copy(Ckk, D), D, RK, A_k, lam_k)) return FitStatus::kNoConvergence;
    return FitStatus::kOk;
  }
  // P = A_v^T C_VK  [RV][D];  M = A_v^T C_VV A_v  [RV][RV]
  std::vector<double> Pm(static_cast<size_t>(RV) * D, 0.0), T(static_cast<size_t>(D) * RV, 0.0),
      M(static_cast<size_t>(RV) * RV, 0.0);
  for (int i = 0; i < D; ++i)
    for (int e = 0; e < RV; ++e) {
      const double ai = A_v[static_cast<size_t>(i) * RV + e];
      for (int j = 0; j < D; ++j) Pm[static_cast<size_t>(e) * D + j] += ai * Cvk[static_cast<size_t>(i) * D + j];
    }
  for (int i = 0; i < D; ++i)
    for (int j = 0; j < D; ++j) {
      const double c = Cvv[static_cast<size_t>(i) * D + j];
      for (int e = 0; e < RV; ++e) T[static_cast<size_t>(i) * RV + e] += c * A_v[static_cast<size_t>(j) * RV + e];
    }
  for (int i = 0; i < D; ++i)
    for (int e = 0; e < RV; ++e) {
      const double ai = A_v[static_cast<size_t>(i) * RV + e];
      for (int e2 = 0; e2 < RV; ++e2) M[static_cast<size_t>(e) * RV + e2] += ai * T[static_cast<size_t>(i) * RV + e2];
    }
  std::vector<double> Wm = Pm;
  if (!spd_solve(M, RV, Wm, D)) return FitStatus::kSingular;
  std::copy(Wm.begin(), Wm.end(), W);
  // R^T R = C_KK - P^T W_pred
  std::vector<double> CR(Ckk, Ckk + dd);
  for (int e = 0; e < RV; ++e)
    for (int i = 0; i < D; ++i) {
      const double pi = Pm[static_cast<size_t>(e) * D + i];
      for (int j = 0; j < D; ++j) CR[static_cast<size_t>(i) * D + j] -= pi * Wm[static_cast<size_t>(e) * D + j];
    }
  if (!top_eigvecs(symmetric_copy(CR.data(), D), D, RK, A_k, lam_k)) return FitStatus::kNoConvergence;
  return FitStatus::kOk;
}

template <int D>
void launch_mfma(const FitArgs& a, int runs, int chunk, hipStream_t s) {
  hipLaunchKernelGGL((moments_mfma_kernel<D>), dim3(runs, a.dm.Hkv), dim3(MomLayout<D>::THREADS), 0, s,
                     static_cast<const uint8_t*>(a.k), static_cast<const uint8_t*>(a.v), a.partial,
                     a.n, a.dm.Hkv, chunk);
}

template <int D>
void launch_valu(const FitArgs& a, int runs, int chunk, hipStream_t s) {
  hipLaunchKernelGGL((moments_valu_kernel<D>), dim3(runs, 3, a.dm.Hkv), dim3(kValuThreads), 0, s,
                     static_cast<const float*>(a.k), static_cast<const float*>(a.v), a.partial, a.n,
                     a.dm.Hkv, chunk);
}

}  // namespace

FitRuns fit_runs(int Hkv, int n) {
  // one workgroup per compute unit (256) over the heads, but at least 2048
  // tokens per run while there are enough tokens (the partials are written
  // and re-read)
  const int max_runs = std::max(1, (kFitGrid + Hkv - 1) / Hkv);
  int runs = std::min(max_runs, std::max(1, n / 2048));
  int chunk = (n + runs - 1) / runs;
  chunk = std::max(kStageTok, (chunk + kStageTok - 1) / kStageTok * kStageTok);
  runs = std::max(1, (n + chunk - 1) / chunk);
  return FitRuns{runs, chunk};
}

hipError_t launch_fit_moments(const FitArgs& a, hipStream_t s) {
  const size_t per_run = static_cast<size_t>(a.dm.Hkv) * 3 * a.dm.D * a.dm.D;
  const unsigned sum_grid = static_cast<unsigned>((per_run + 255) / 256);
  if (a.n == 0) {
    if (!a.accumulate) return launch_zero_fill(a.moments, per_run * sizeof(double), s);
    return hipSuccess;
  }
  const FitRuns fr = fit_runs(a.dm.Hkv, a.n);
  if (a.dm.dtype == 0) {
    if (a.dm.D == 128) launch_mfma<128>(a, fr.runs, fr.chunk, s);
    else launch_mfma<64>(a, fr.runs, fr.chunk, s);
  } else {
    if (a.dm.D == 128) launch_valu<128>(a, fr.runs, fr.chunk, s);
    else launch_valu<64>(a, fr.runs, fr.chunk, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moments_sum_kernel, dim3(sum_grid), dim3(256), 0, s, a.partial, a.moments,
                     fr.runs, a.dm.D, per_run, a.accumulate);
  return hipGetLastError();
}

FitStatus fit_solve(const Dims& dm, const double* moments, double* A_v, double* A_k, double* W,
                    double* lam_v, double* lam_k) {
  const int H = dm.Hkv, D = dm.D, RV = dm.RV, RK = dm.RK;
  const size_t dd = static_cast<size_t>(D) * D;
  std::vector<FitStatus> st(H, FitStatus::kOk);
  auto work = [&](int g) {
    st[g] = solve_head(dm, moments + static_cast<size_t>(g) * 3 * dd,
                       A_v + static_cast<size_t>(g) * D * RV, A_k + static_cast<size_t>(g) * D * RK,
                       dm.exact ? W + static_cast<size_t>(g) * RV * D : nullptr,
                       lam_v ? lam_v + static_cast<size_t>(g) * RV : nullptr,
                       lam_k ? lam_k + static_cast<size_t>(g) * RK : nullptr);
  };
  const int workers = std::min(H, 16);
  if (workers <= 1) {
    for (int g = 0; g < H; ++g) work(g);
  } else {
    std::vector<std::thread> pool;
    for (int t = 0; t < workers; ++t)
      pool.emplace_back([&, t] {
        for (int g = t; g < H; g += workers) work(g);
      });
    for (auto& th : pool) th.join();
  }
  for (FitStatus s : st)
    if (s != FitStatus::kOk) return s;
  return FitStatus::kOk;
}

}  // namespace kvlr
