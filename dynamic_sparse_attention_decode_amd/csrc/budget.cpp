// Profiling-guided speculation budget (PRR abstract: a profiling-guided speculation budget keeps speculative work
// off the critical path; PRR summary page, Limitations: overhead estimates come from profiled grids and polynomial
// regression for context lengths outside the grid).
//
// Speculation runs concurrently with selection, so it stays off the critical path while its time does not exceed the
// selection time. The budget is the largest profiled K' whose measured speculation time fits under the selection time
// at the target block count; off the profiled grid that selection time comes from a least-squares polynomial in the
// block count (abscissae scaled to [0, 1], normal equations, Gaussian elimination with partial pivoting).
#include <math.h>
#include <stdint.h>

#include "../../include/prr.h"

namespace {

bool lstsq_poly(const double* x, const double* y, int n, int deg, double xs, double* coef) {
  double A[5][6] = {};
  for (int i = 0; i < n; ++i) {
    double p[9];
    p[0] = 1.0;
    const double t = x[i] / xs;
    for (int k = 1; k <= 2 * deg; ++k) p[k] = p[k - 1] * t;
    for (int r = 0; r <= deg; ++r) {
      for (int c = 0; c <= deg; ++c) A[r][c] += p[r + c];
      A[r][deg + 1] += p[r] * y[i];
    }
  }
  const int m = deg + 1;
  for (int c = 0; c < m; ++c) {
    int piv = c;
    for (int r = c + 1; r < m; ++r)
      if (fabs(A[r][c]) > fabs(A[piv][c])) piv = r;
    if (fabs(A[piv][c]) < 1e-300) return false;
    if (piv != c)
      for (int k = 0; k <= m; ++k) { const double t = A[c][k]; A[c][k] = A[piv][k]; A[piv][k] = t; }
    for (int r = 0; r < m; ++r) {
      if (r == c) continue;
      const double f = A[r][c] / A[c][c];
      for (int k = c; k <= m; ++k) A[r][k] -= f * A[c][k];
    }
  }
  for (int r = 0; r < m; ++r) coef[r] = A[r][m] / A[r][r];
  return true;
}

}  // namespace

extern "C" int32_t prr_choose_budget(const double* n_grid, const double* t_sel, int32_t n_pts_sel,
                                     const double* kspec_grid, const double* t_spec, int32_t n_pts_spec,
                                     double n_target, int32_t poly_degree) {
  if (!n_grid || !t_sel || n_pts_sel < 1 || n_pts_spec < 0 || (n_pts_spec > 0 && (!kspec_grid || !t_spec)))
    return -1;
  double t_target = 0.0;
  bool on_grid = false;
  for (int i = 0; i < n_pts_sel; ++i)
    if (n_grid[i] == n_target) { t_target = t_sel[i]; on_grid = true; break; }
  if (!on_grid) {
    int deg = poly_degree < 0 ? 0 : poly_degree;
    if (deg > 4) deg = 4;
    if (deg > n_pts_sel - 1) deg = n_pts_sel - 1;
    double xs = 0.0;
    for (int i = 0; i < n_pts_sel; ++i) xs = fmax(xs, fabs(n_grid[i]));
    if (xs == 0.0) xs = 1.0;
    double c[5] = {};
    if (!lstsq_poly(n_grid, t_sel, n_pts_sel, deg, xs, c)) return -1;
    const double t = n_target / xs;
    double p = 1.0;
    for (int k = 0; k <= deg; ++k) { t_target += c[k] * p; p *= t; }
  }
  int32_t best = 0;
  for (int i = 0; i < n_pts_spec; ++i)
    if (t_spec[i] <= t_target && kspec_grid[i] > best) best = (int32_t)kspec_grid[i];
  return best;
}

// The fused single-stream step co-schedules the speculation with the selection launch, so speculation is off the
// critical path exactly when the step with it is no slower than the step without it: the budget is the largest
// profiled K' whose measured step time is at most that of K' = 0 (which the grid must hold).
extern "C" int32_t prr_choose_budget_fused(const double* kspec_grid, const double* t_step, int32_t n_pts) {
  if (!kspec_grid || !t_step || n_pts < 1) return -1;
  int zero = -1;
  for (int i = 0; i < n_pts; ++i) {
    if (!(kspec_grid[i] >= 0.0) || !isfinite(t_step[i])) return -1;
    if (kspec_grid[i] == 0.0 && zero < 0) zero = i;
  }
  if (zero < 0) return -1;
  const double t0 = t_step[zero];
  int32_t best = 0;
  for (int i = 0; i < n_pts; ++i)
    if (t_step[i] <= t0 && kspec_grid[i] > best) best = (int32_t)kspec_grid[i];
  return best;
}
