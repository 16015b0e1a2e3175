// Hardware-aware recomputation ratio -- "Adaptive KV Cache Reuse for Fast
// Long-Context LLM Serving" (CacheTune), App. C.1 (per-token recomputation and
// loading costs) and App. C.2 (golden-section search on the measured latency,
// warm-started by the cost model).  Host logic only: the caller measures.
#include <cmath>
#include <string>

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
