// Head-wise budget redistribution ("HeSS: Head Sensitivity Score for
// Sparsity Redistribution in VGGT", proposed method: the layer's attention
// budget is reallocated across heads by iterative capping).
//
// Keep fractions kappa_h = 1 - rho_h solve
//   kappa_h = clamp(lambda * w_h, lo, hi),  sum_h kappa_h = H * target,
// with lo = 1 - rho_max, hi = 1 - rho_min, target = 1 - mean_rho.  The sum is
// continuous and non-decreasing in lambda (strictly increasing while any head
// is unclipped), running from H * lo to H * hi, so the kappa vector is unique.
//
// Method: bisection on lambda brackets the solution to float64 resolution;
// the heads are then split into those clipped low, clipped high and free at
// that lambda, and lambda is re-solved exactly on the free heads (the
// iterative-capping step).  If the exact re-solve moves a free head across a
// bound (possible only within rounding of a breakpoint), that head is clipped
// and the step repeats.
#include <math.h>

#include <vector>

#include "bsga_internal.hpp"

namespace {

double clampd(double x, double lo, double hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace

int bsga_redistribute(int32_t heads, const double* weights, double mean_rho, double rho_min,
                      double rho_max, double* rho_out) {
  if (!weights || !rho_out || heads < 1 || heads > BSGA_MAX_HEADS) return BSGA_ERR_INVALID_ARG;
  if (!(rho_min >= 0.0) || !(rho_min <= mean_rho) || !(mean_rho <= rho_max) || !(rho_max <= 1.0))
    return BSGA_ERR_INVALID_ARG;
  for (int h = 0; h < heads; ++h)
    if (!(weights[h] > 0.0) || !isfinite(weights[h])) return BSGA_ERR_INVALID_ARG;
  const double lo = 1.0 - rho_max, hi = 1.0 - rho_min, target = 1.0 - mean_rho;
  const double total = target * heads;
  if (hi - lo <= 0.0) {  // a single admissible value
    for (int h = 0; h < heads; ++h) rho_out[h] = mean_rho;
    return BSGA_OK;
  }
  auto sum_at = [&](double lam) {
    double s = 0.0;
    for (int h = 0; h < heads; ++h) s += clampd(lam * weights[h], lo, hi);
    return s;
  };
  // bracket: at lam_lo every head sits at or below lo, at lam_hi every head
  // at or above hi
  double wmin = weights[0], wmax = weights[0];
  for (int h = 1; h < heads; ++h) {
    wmin = fmin(wmin, weights[h]);
    wmax = fmax(wmax, weights[h]);
  }
  double a = lo / wmax, b = hi / wmin;
  for (int it = 0; it < 200 && b > a; ++it) {
    const double m = 0.5 * (a + b);
    if (m <= a || m >= b) break;
    if (sum_at(m) < total) a = m; else b = m;
  }
  // iterative capping at the bracketed lambda: clip, re-solve the free heads
  std::vector<int> state(heads);  // -1 clipped low, +1 clipped high, 0 free
  const double lam0 = 0.5 * (a + b);
  for (int h = 0; h < heads; ++h) {
    const double x = lam0 * weights[h];
    state[h] = x <= lo ? -1 : (x >= hi ? 1 : 0);
  }
  std::vector<double> kappa(heads);
  for (int round = 0; round <= heads; ++round) {
    double rest = total, wfree = 0.0;
    for (int h = 0; h < heads; ++h) {
      if (state[h] < 0) rest -= lo;
      else if (state[h] > 0) rest -= hi;
      else wfree += weights[h];
    }
    bool moved = false;
    if (wfree > 0.0) {
      const double lam = rest / wfree;
      for (int h = 0; h < heads; ++h) {
        if (state[h] != 0) continue;
        const double x = lam * weights[h];
        if (x < lo) { state[h] = -1; moved = true; }
        else if (x > hi) { state[h] = 1; moved = true; }
        else kappa[h] = x;
      }
    }
    if (!moved) break;
  }
  for (int h = 0; h < heads; ++h) {
    if (state[h] < 0) kappa[h] = lo;
    else if (state[h] > 0) kappa[h] = hi;
    rho_out[h] = clampd(1.0 - kappa[h], rho_min, rho_max);
  }
  return BSGA_OK;
}
