// Host float64 solve of the joint decoder fit's normal equations.
//
// BasisKV: Value Latents for Communication and Key Routing, English abstract
// (factors optimised jointly across the per-GPU attention partitions against
// the complete attention output): the joint decoder is the least-squares
// solution D of (Z^T Z) D = Z^T X, with the moments formed on the GPU.
//
// Cholesky Z^T Z = L L^T by blocks of 64 columns (each block's diagonal
// factor, then its panel below, then the trailing update, rows split over host
// threads); then L Y = Z^T X and L^T D = Y over blocks of 256 right-hand-side
// columns (one host thread each), rows taken 32 at a time and updated from
// the solved rows 64 at a time, so that the rows in use stay in cache.
// The row updates run in an AVX2/FMA build of the same loop where the CPU has
// those units (checked at run time), else in the baseline build.

#include <math.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "kvlr_host.h"

namespace kvlr {
namespace {

// Runs fn(t) for t in [0, n) on up to 16 host threads (fn(0) on this one).
template <class Fn>
void parallel_for(int n, Fn fn) {
  const int nthreads =
      std::max(1, std::min<int>({16, n, static_cast<int>(std::thread::hardware_concurrency())}));
  auto run = [&](int t0) {
    for (int t = t0; t < n; t += nthreads) fn(t);
  };
  std::vector<std::thread> pool;
  for (int t = 1; t < nthreads; ++t) pool.emplace_back(run, t);
  run(0);
  for (auto& th : pool) th.join();
}

// acc[0 .. w) -= sum_j coef[j] * rows[j][0 .. w) over nrows rows spaced
// `stride` doubles apart, four rows a pass.
inline void rows_update(double* acc, const double* coef, const double* rows, size_t nrows,
                        size_t stride, size_t w) {
  size_t j = 0;
  for (; j + 4 <= nrows; j += 4) {
    const double l0 = coef[j], l1 = coef[j + 1], l2 = coef[j + 2], l3 = coef[j + 3];
    const double* y0 = rows + j * stride;
    const double* y1 = y0 + stride;
    const double* y2 = y1 + stride;
    const double* y3 = y2 + stride;
    for (size_t c = 0; c < w; ++c) acc[c] -= (l0 * y0[c] + l1 * y1[c]) + (l2 * y2[c] + l3 * y3[c]);
  }
  for (; j < nrows; ++j) {
    const double l = coef[j];
    const double* y = rows + j * stride;
    for (size_t c = 0; c < w; ++c) acc[c] -= l * y[c];
  }
}

__attribute__((target("avx2,fma"))) void rows_update_avx2(double* acc, const double* coef,
                                                           const double* rows, size_t nrows,
                                                           size_t stride, size_t w) {
  rows_update(acc, coef, rows, nrows, stride, w);
}

void rows_update_base(double* acc, const double* coef, const double* rows, size_t nrows,
                      size_t stride, size_t w) {
  rows_update(acc, coef, rows, nrows, stride, w);
}

using RowsUpdate = void (*)(double*, const double*, const double*, size_t, size_t, size_t);

RowsUpdate pick_rows_update() {
#if defined(__x86_64__)
  __builtin_cpu_init();
  if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma")) return rows_update_avx2;
#endif
  return rows_update_base;
}

}  // namespace

FitStatus joint_solve(int nl, int nx, const double* zz, const double* zx, double* D) {
  constexpr int kNb = 64;
  const size_t n = static_cast<size_t>(nl);
  std::vector<double> L(n * n, 0.0);  // lower triangle; the trailing update works in place
  double dmax = 0.0;
  for (int i = 0; i < nl; ++i) dmax = std::max(dmax, zz[static_cast<size_t>(i) * n + i]);
  if (!(dmax > 0.0)) return FitStatus::kSingular;
  for (size_t i = 0; i < n; ++i)
    for (size_t j = 0; j <= i; ++j) L[i * n + j] = zz[i * n + j];
  for (int j0 = 0; j0 < nl; j0 += kNb) {
    const int j1 = std::min(nl, j0 + kNb);
    // diagonal block, left-looking within it (earlier blocks are already applied)
    for (int j = j0; j < j1; ++j) {
      double* Lj = &L[j * n];
      double s = Lj[j];
      for (int k = j0; k < j; ++k) s -= Lj[k] * Lj[k];
      if (!(s > 1e-12 * dmax)) return FitStatus::kSingular;
      const double djj = sqrt(s);
      Lj[j] = djj;
      const double inv = 1.0 / djj;
      for (int i = j + 1; i < j1; ++i) {
        double* Li = &L[i * n];
        double t = Li[j];
        for (int k = j0; k < j; ++k) t -= Li[k] * Lj[k];
        Li[j] = t * inv;
      }
    }
    const int rows = nl - j1;
    const int nblk = (rows + kNb - 1) / kNb;
    // the panel below the block (rows >= j1, columns j0 .. j1-1), then the
    // trailing lower triangle: L[i][c] -= L[i][j0 .. j1) . L[c][j0 .. j1)
    parallel_for(nblk, [&](int rb) {
      const int r0 = j1 + rb * kNb, r1 = std::min(nl, r0 + kNb);
      for (int i = r0; i < r1; ++i) {
        double* Li = &L[i * n];
        for (int j = j0; j < j1; ++j) {
          const double* Lj = &L[j * n];
          double t = Li[j];
          for (int k = j0; k < j; ++k) t -= Li[k] * Lj[k];
          Li[j] = t / Lj[j];
        }
      }
    });
    parallel_for(nblk, [&](int rb) {
      const int r0 = j1 + rb * kNb, r1 = std::min(nl, r0 + kNb);
      for (int i = r0; i < r1; ++i) {
        double* Li = &L[i * n];
        for (int c = j1; c <= i; ++c) {
          const double* Lc = &L[c * n];
          double t = 0.0;
          for (int k = j0; k < j1; ++k) t += Li[k] * Lc[k];
          Li[c] -= t;
        }
      }
    });
  }
  // U = L^T by rows, for the back substitution's coefficients
  std::vector<double> U(n * n, 0.0);
  for (size_t i = 0; i < n; ++i)
    for (size_t j = 0; j <= i; ++j) U[j * n + i] = L[i * n + j];
  const RowsUpdate update = pick_rows_update();
  // Substitutions over a column block [c0, c0 + w) of the right-hand sides,
  // rows in blocks of kRb: a block's rows are first updated from every row
  // already solved (those rows taken kKb at a time, so each stays in cache
  // while the block's rows use it), then solved among themselves.
  constexpr size_t kCols = 256, kRb = 32, kKb = 64;
  parallel_for(static_cast<int>((static_cast<size_t>(nx) + kCols - 1) / kCols), [&](int blk) {
    const size_t c0 = static_cast<size_t>(blk) * kCols;
    const size_t w = std::min(static_cast<size_t>(nx), c0 + kCols) - c0;
    const size_t sx = static_cast<size_t>(nx);
    std::vector<double> A(kRb * kCols);
    // L Y = zx, rows top to bottom
    for (size_t i0 = 0; i0 < n; i0 += kRb) {
      const size_t nb = std::min(kRb, n - i0);
      for (size_t r = 0; r < nb; ++r)
        for (size_t c = 0; c < w; ++c) A[r * kCols + c] = zx[(i0 + r) * sx + c0 + c];
      for (size_t k0 = 0; k0 < i0; k0 += kKb) {
        const size_t kn = std::min(kKb, i0 - k0);
        for (size_t r = 0; r < nb; ++r)
          update(&A[r * kCols], &L[(i0 + r) * n + k0], &D[k0 * sx + c0], kn, sx, w);
      }
      for (size_t r = 0; r < nb; ++r) {
        update(&A[r * kCols], &L[(i0 + r) * n + i0], &A[0], r, kCols, w);
        const double inv = 1.0 / L[(i0 + r) * n + i0 + r];
        for (size_t c = 0; c < w; ++c) A[r * kCols + c] *= inv;
      }
      for (size_t r = 0; r < nb; ++r)
        for (size_t c = 0; c < w; ++c) D[(i0 + r) * sx + c0 + c] = A[r * kCols + c];
    }
    // L^T D = Y, rows bottom to top (block rows i0 .. i0 + nb - 1, solved from the last)
    for (size_t end = n; end > 0;) {
      const size_t nb = std::min(kRb, end);
      const size_t i0 = end - nb;
      for (size_t r = 0; r < nb; ++r)
        for (size_t c = 0; c < w; ++c) A[r * kCols + c] = D[(i0 + r) * sx + c0 + c];
      for (size_t k0 = end; k0 < n; k0 += kKb) {
        const size_t kn = std::min(kKb, n - k0);
        for (size_t r = 0; r < nb; ++r)
          update(&A[r * kCols], &U[(i0 + r) * n + k0], &D[k0 * sx + c0], kn, sx, w);
      }
      for (size_t r = nb; r-- > 0;) {
        update(&A[r * kCols], &U[(i0 + r) * n + i0 + r + 1], &A[(r + 1) * kCols], nb - r - 1, kCols, w);
        const double inv = 1.0 / U[(i0 + r) * n + i0 + r];
        for (size_t c = 0; c < w; ++c) A[r * kCols + c] *= inv;
      }
      for (size_t r = 0; r < nb; ++r)
        for (size_t c = 0; c < w; ++c) D[(i0 + r) * sx + c0 + c] = A[r * kCols + c];
      end = i0;
    }
  });
  return FitStatus::kOk;
}

}  // namespace kvlr
