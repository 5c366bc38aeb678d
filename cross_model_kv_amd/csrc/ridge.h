// Host ridge solve (plain C++, no HIP).
#pragma once

namespace kvmap {

// W = (sym(M_xx) + lambda I)^-1 M_xy and b = mean_y - mean_x W in float64, M_xx read from its
// upper triangle; W_out written output-major [q][p].  Returns 0 on success, 1 if the
// Cholesky factorisation meets a non-positive pivot.
int ridge_solve_f64(int p, int q, const float* mean_x, const float* mean_y, const float* M_xx,
                    const float* M_xy, double lambda, float* W_out, float* b_out,
                    int n_threads);

}  // namespace kvmap
