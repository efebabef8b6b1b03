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
//    one KV head; wave w owns the 16-dimension row block w of all three
//    moments. Tokens are staged 64 at a time into LDS directly in matrix-core
//    fragment order (8 tokens of one dimension per lane), so each operand is
//    one 16-byte LDS read, and v_mfma_f32_16x16x32_bf16 forms the products
//    (exact for bf16) with float32 sums. The next 64 tokens' loads are in
//    flight while the current ones are multiplied.
//  - moments_valu_kernel (f32 samples): the same partial sums on the vector
//    ALUs, one 8x8 (or 4x4) block of one moment per thread.
//  - moments_sum_kernel adds the per-run partials in a fixed order into
//    float64 moments (optionally onto what the buffer already holds).
//  - The host solves the small symmetric eigenproblems in float64:
//    Householder reduction to tridiagonal form, then implicit QR steps with
//    the Wilkinson shift (Golub and Van Loan, Matrix Computations, the
//    symmetric QR algorithm), eigenvectors accumulated throughout.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "kvlr_device.h"
#include "kvlr_internal.h"

namespace kvlr {
namespace {

constexpr int kStageTok = 64;  // tokens staged per LDS fill

template <int D>
struct MomLayout {
  static constexpr int NB = D / 16;                    // 16-dimension blocks = waves
  static constexpr int THREADS = NB * kWave;
  static constexpr int KSTEPS = kStageTok / 32;        // 32-token matrix-core k-steps
  static constexpr int FRAG_DW = kWave * 4;            // one fragment: 64 lanes x 16 bytes
  static constexpr int RB_DW = KSTEPS * FRAG_DW + 4;   // +16 bytes: blocks start on rotating banks
  static constexpr int TENSOR_DW = NB * RB_DW;
  static constexpr int TOTAL_DW = 2 * TENSOR_DW;       // V then K
  static constexpr int CHUNKS = D / 8;                 // 16-byte chunks per token row
  static_assert(2 * 16 * CHUNKS == THREADS, "one staging task per thread");
};

// bf16 half e (0..7) of a 16-byte chunk
__device__ __forceinline__ uint32_t half_of(const uint4& x, int e) {
  const uint32_t w = e < 2 ? x.x : (e < 4 ? x.y : (e < 6 ? x.z : x.w));
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

template <int D>
__global__ __launch_bounds__(MomLayout<D>::THREADS) void moments_mfma_kernel(
    const uint8_t* __restrict__ k, const uint8_t* __restrict__ v, float* __restrict__ partial,
    int n, int Hkv, int chunk_tokens) {
  using L = MomLayout<D>;
  __shared__ __align__(16) uint32_t lds[L::TOTAL_DW];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;  // row block
  const int c = blockIdx.x, g = blockIdx.y;
  const int t0 = c * chunk_tokens;
  const int t1 = min(t0 + chunk_tokens, n);
  const size_t row_bytes = static_cast<size_t>(Hkv) * D * 2;

  // staging task: tensor tt, 4-token group tg, 16-byte chunk ch
  const int ch = tid % L::CHUNKS;
  const int tg = (tid / L::CHUNKS) % 16;
  const int tt = tid / (16 * L::CHUNKS);
  const uint8_t* src = (tt == 0 ? v : k) + static_cast<size_t>(g) * D * 2 + ch * 16;
  // LDS slot of (token 4*tg + u, dimension 8*ch + e): block ch/2, k-step tg/8,
  // lane (tg%8)/2 * 16 + (ch%2)*8 + e, tokens 4*(tg%2) .. +3 of the lane's 8
  const int slot_dw = tt * L::TENSOR_DW + (ch / 2) * L::RB_DW + (tg / 8) * L::FRAG_DW +
                      (((tg % 8) / 2) * 16 + (ch % 2) * 8) * 4 + 2 * (tg % 2);

  uint4 x[4];
  auto load_stage = [&](int base) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = base + 4 * tg + u;
      const int tc = min(t, t1 - 1);
      x[u] = load16(src + static_cast<size_t>(tc) * row_bytes);
      if (t >= t1) x[u] = make_uint4(0, 0, 0, 0);
    }
  };

  f32x4 acc[3][L::NB];
#pragma unroll
  for (int m = 0; m < 3; ++m)
#pragma unroll
    for (int j = 0; j < L::NB; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (t0 < t1) load_stage(t0);
  for (int base = t0; base < t1; base += kStageTok) {
    __syncthreads();  // the previous stage's fragments have been read
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint2 pk;
      pk.x = half_of(x[0], e) | (half_of(x[1], e) << 16);
      pk.y = half_of(x[2], e) | (half_of(x[3], e) << 16);
      *reinterpret_cast<uint2*>(&lds[slot_dw + e * 4]) = pk;
    }
    __syncthreads();
    if (base + kStageTok < t1) load_stage(base + kStageTok);
#pragma unroll
    for (int ks = 0; ks < L::KSTEPS; ++ks) {
      const int off = ks * L::FRAG_DW + lane * 4;
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(&lds[wv * L::RB_DW + off]);
      const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&lds[L::TENSOR_DW + wv * L::RB_DW + off]);
#pragma unroll
      for (int j = 0; j < L::NB; ++j) {
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&lds[j * L::RB_DW + off]);
        const bf16x8 bk = *reinterpret_cast<const bf16x8*>(&lds[L::TENSOR_DW + j * L::RB_DW + off]);
        acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[0][j], 0, 0, 0);
        acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bk, acc[1][j], 0, 0, 0);
        acc[2][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bk, acc[2][j], 0, 0, 0);
      }
    }
  }
  // lane holds rows 4*(lane/16) + r of column lane%16 of each 16x16 tile
  const int kq = lane >> 4, col = lane & 15;
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    float* out = partial + ((static_cast<size_t>(c) * Hkv + g) * 3 + m) * D * D;
#pragma unroll
    for (int j = 0; j < L::NB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        out[static_cast<size_t>(wv * 16 + 4 * kq + r) * D + j * 16 + col] = acc[m][j][r];
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

__global__ __launch_bounds__(256) void moments_sum_kernel(const float* __restrict__ partial,
                                                          double* __restrict__ moments, int runs,
                                                          size_t per_run, int accumulate) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= per_run) return;
  double s = accumulate ? moments[i] : 0.0;
  for (int c = 0; c < runs; ++c) s += static_cast<double>(partial[static_cast<size_t>(c) * per_run + i]);
  moments[i] = s;
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
  // about 512 workgroups over the heads, but at least 2048 tokens per run
  // while there are enough tokens (the partials are written and re-read)
  const int max_runs = std::max(1, (512 + Hkv - 1) / Hkv);
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
                     fr.runs, per_run, a.accumulate);
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
