// Hardware-aware recomputation ratio -- "Adaptive KV Cache Reuse for Fast
// Long-Context LLM Serving" (CacheTune), App. C.1 (per-token recomputation and
// loading costs, fixed per-layer overhead) and App. C.2 (golden-section search
// on the measured latency, warm-started by the cost model).  Host logic only:
// the caller measures.
#include <algorithm>
#include <cmath>
#include <string>
#include <vector>

#include "ct_internal.h"

extern "C" ct_status cachetune_calibrate_ratio(double t_c, double t_i, double r_min, double r_max,
                                               double half_width, double eps, ct_cost_fn cost,
                                               void* user, double* r_out, int32_t* n_probes) {
  using ct::fail;
  if (!(std::isfinite(t_c) && std::isfinite(t_i)) || t_c < 0.0 || t_i < 0.0 || t_c + t_i <= 0.0)
    return fail(CT_E_INVALID, "calibrate_ratio: t_c and t_i must be finite, >= 0 and not both 0");
  if (!(r_min >= 0.0 && r_max <= 1.0 && r_min <= r_max))
    return fail(CT_E_INVALID, "calibrate_ratio: need 0 <= r_min <= r_max <= 1");
  if (!(half_width > 0.0) || !(eps > 0.0))
    return fail(CT_E_INVALID, "calibrate_ratio: half_width and eps must be > 0");
  if (!cost || !r_out) return fail(CT_E_INVALID, "calibrate_ratio: NULL callback or output");

  // warm start: recomputing r*N tokens and loading (1 - r)*N take equal time
  double r0 = t_i / (t_c + t_i);
  r0 = r0 < r_min ? r_min : (r0 > r_max ? r_max : r0);
  double a = r0 - half_width < r_min ? r_min : r0 - half_width;
  double b = r0 + half_width > r_max ? r_max : r0 + half_width;

  const double phi = (std::sqrt(5.0) - 1.0) / 2.0;
  int32_t calls = 0;
  auto eval = [&](double r, double* f) -> bool {
    *f = cost(r, user);
    ++calls;
    return std::isfinite(*f);
  };
  double x1 = b - phi * (b - a), x2 = a + phi * (b - a);
  double f1, f2;
  if (!eval(x1, &f1) || !eval(x2, &f2)) {
    if (n_probes) *n_probes = calls;
    return fail(CT_E_INVALID, "calibrate_ratio: the cost callback returned a non-finite value");
  }
  while (b - a >= eps) {
    if (f1 <= f2) {  // the minimum lies in [a, x2]; x1 becomes the new upper probe
      b = x2;
      x2 = x1;
      f2 = f1;
      x1 = b - phi * (b - a);
      if (!eval(x1, &f1)) break;
    } else {  // the minimum lies in [x1, b]; x2 becomes the new lower probe
      a = x1;
      x1 = x2;
      f1 = f2;
      x2 = a + phi * (b - a);
      if (!eval(x2, &f2)) break;
    }
  }
  if (n_probes) *n_probes = calls;
  if (!(std::isfinite(f1) && std::isfinite(f2)))
    return fail(CT_E_INVALID, "calibrate_ratio: the cost callback returned a non-finite value");
  *r_out = 0.5 * (a + b);
  return CT_OK;
}

// App. C.1 cost model fitted to measured request times.  Per layer the
// pipeline overlaps the recomputation of r*N tokens (t_c each) with the
// loading of the other (1 - r)*N (t_i each), so the longer path sets the
// layer's time, plus a fixed per-layer overhead t_o:
//   T(r) = L * (t_o + max(r*N*t_c, (1 - r)*N*t_i)).
// Probes sorted by r are split into a lower (loading-bound) and an upper
// (recomputation-bound) part of at least two probes each (one probe would fit
// any slope exactly); for each split the three costs
// solve the linear least-squares problem of that assignment (normal
// equations, Gaussian elimination with partial pivoting).  A split counts when
// t_c and t_i come out positive and t_o non-negative and every probe lies on
// its assigned side of the balance ratio t_i / (t_c + t_i); the split with the
// smallest squared residual is kept (the lower split on a tie).
namespace {
bool solve3(double A[3][3], double y[3], double x[3]) {
  for (int c = 0; c < 3; ++c) {
    int p = c;
    for (int r = c + 1; r < 3; ++r)
      if (std::fabs(A[r][c]) > std::fabs(A[p][c])) p = r;
    if (!(std::fabs(A[p][c]) > 0.0)) return false;
    if (p != c) {
      for (int k = 0; k < 3; ++k) std::swap(A[c][k], A[p][k]);
      std::swap(y[c], y[p]);
    }
    for (int r = c + 1; r < 3; ++r) {
      const double f = A[r][c] / A[c][c];
      for (int k = c; k < 3; ++k) A[r][k] -= f * A[c][k];
      y[r] -= f * y[c];
    }
  }
  for (int c = 2; c >= 0; --c) {
    double s = y[c];
    for (int k = c + 1; k < 3; ++k) s -= A[c][k] * x[k];
    x[c] = s / A[c][c];
  }
  return true;
}
}  // namespace

extern "C" ct_status cachetune_fit_cost_model(const double* r, const double* t, int32_t n, int32_t L,
                                              int32_t N, double* t_c, double* t_i, double* t_o) {
  using ct::fail;
  if (!r || !t || !t_c || !t_i || !t_o) return fail(CT_E_INVALID, "fit_cost_model: NULL argument");
  if (n < 4 || n > 1024) return fail(CT_E_INVALID, "fit_cost_model: need 4 to 1024 probes");
  if (L < 1 || N < 1) return fail(CT_E_INVALID, "fit_cost_model: L and N must be positive");
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) {
    if (!(std::isfinite(r[i]) && std::isfinite(t[i])) || r[i] < 0.0 || r[i] > 1.0)
      return fail(CT_E_INVALID, "fit_cost_model: ratios must lie in [0, 1], times must be finite");
    order[i] = i;
  }
  std::sort(order.begin(), order.end(), [&](int a, int b) { return r[a] < r[b] || (r[a] == r[b] && a < b); });
  bool found = false;
  double best = 0.0, best_x[3] = {0.0, 0.0, 0.0};
  for (int k = 2; k <= n - 2; ++k) {  // probes order[0 .. k) loading-bound, the rest recomputation-bound
    // unknowns (t_o, t_c, t_i); row i: t[i] / L = t_o + [r N] t_c  or  t_o + [(1 - r) N] t_i
    double A[3][3] = {{0, 0, 0}, {0, 0, 0}, {0, 0, 0}}, y[3] = {0, 0, 0};
    for (int p = 0; p < n; ++p) {
      const int i = order[p];
      const double row[3] = {1.0, p >= k ? r[i] * N : 0.0, p < k ? (1.0 - r[i]) * N : 0.0};
      const double b = t[i] / L;
      for (int a = 0; a < 3; ++a) {
        y[a] += row[a] * b;
        for (int c = 0; c < 3; ++c) A[a][c] += row[a] * row[c];
      }
    }
    double x[3];
    if (!solve3(A, y, x)) continue;
    const double to = x[0], tc = x[1], ti = x[2];
    if (!(tc > 0.0 && ti > 0.0 && to >= 0.0)) continue;
    const double rb = ti / (tc + ti);
    bool ok = true;
    for (int p = 0; p < n && ok; ++p) ok = p < k ? r[order[p]] <= rb : r[order[p]] >= rb;
    if (!ok) continue;
    double res = 0.0;
    for (int p = 0; p < n; ++p) {
      const int i = order[p];
      const double model = L * (to + std::max(r[i] * N * tc, (1.0 - r[i]) * N * ti));
      res += (t[i] - model) * (t[i] - model);
    }
    if (!found || res < best) {
      found = true;
      best = res;
      best_x[0] = to;
      best_x[1] = tc;
      best_x[2] = ti;
    }
  }
  if (!found) return fail(CT_E_INVALID, "fit_cost_model: the probes do not show a loading-bound and a recomputation-bound part");
  *t_o = best_x[0];
  *t_c = best_x[1];
  *t_i = best_x[2];
  return CT_OK;
}
