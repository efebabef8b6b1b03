// Host-only interfaces shared by the HIP sources and the plain C++ host solve.
#pragma once

namespace kvlr {

enum class FitStatus { kOk, kSingular, kNoConvergence };

// Host: D [nl][nx] = zz^-1 zx for the symmetric positive definite zz [nl][nl]
// (float64, row-major); kSingular when a Cholesky pivot falls to 1e-12 of the
// largest diagonal entry.
FitStatus joint_solve(int nl, int nx, const double* zz, const double* zx, double* D);

}  // namespace kvlr
