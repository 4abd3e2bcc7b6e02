// Chunk-aware growth (CAG) of the sparsity ratio over the chunks of an
// autoregressive rollout (Light Forcing §2.1: the first chunk is attended
// densely, later chunks progressively more sparsely, s_i = s_base -
// alpha_i * beta with alpha_i following the noise level as 1/sqrt, and beta
// chosen so that the total attention FLOPs match a target sparsity).
//
// Host code.  Chunk 0 has s_0 = 0; chunk i >= 1 has
// s_i = clip(s_base - beta / sqrt(i + 1), 0, s_max).  The kept cost
// K(beta) = sum_i (1 - s_i) cost_i (ascending i) never decreases with beta;
// beta is the upper end of a fixed bisection (200 halvings at most) of a
// bracket that clips every s_i at s_max at one end and at 0 at the other, so
// K(beta) reaches (1 - s_target) * sum_i cost_i.  All arithmetic is float64
// in a fixed order without contraction, so results are reproducible bit for
// bit.  Frame budgets: k_i = floor((1 - s_i) * c_i + 1/2) clipped to [1, c_i].
#pragma STDC FP_CONTRACT OFF
#pragma clang fp contract(off)

#include <cmath>

#include "fsa_internal.h"

namespace {

struct Schedule {
  int n;
  const double *cost;
  double s_base, s_max;

  double sparsity(double beta, int i) const {
    if (i == 0) return 0.0;
    const double v = s_base - (1.0 / std::sqrt(i + 1.0)) * beta;
    const double lo = v > 0.0 ? v : 0.0;
    return lo < s_max ? lo : s_max;
  }
  double kept(double beta) const {
    double acc = 0.0;
    for (int i = 0; i < n; ++i) acc = acc + (1.0 - sparsity(beta, i)) * cost[i];
    return acc;
  }
};

}  // namespace

extern "C" fsa_status fsa_cag_schedule(int32_t n_chunks, const double *cost, double s_target,
                                       double s_base, double s_max, const int32_t *candidates,
                                       double *sparsity, int32_t *budgets, double *beta_out) {
  fsa::clear_error();
  FSA_REQUIRE(n_chunks >= 1, FSA_E_ARG, "n_chunks=%d must be >= 1", n_chunks);
  FSA_REQUIRE(cost && sparsity, FSA_E_ARG, "null pointer argument");
  FSA_REQUIRE(s_target >= 0.0 && s_target < 1.0 && s_max >= 0.0 && s_max < 1.0 &&
                  s_base >= 0.0 && s_base <= 1.0,
              FSA_E_ARG, "ratios out of range (s_target, s_max in [0, 1), s_base in [0, 1])");
  double total = 0.0;
  for (int i = 0; i < n_chunks; ++i) {
    FSA_REQUIRE(cost[i] > 0.0 && std::isfinite(cost[i]), FSA_E_ARG,
                "cost[%d] must be positive and finite", i);
    total = total + cost[i];
  }
  if (budgets) {
    FSA_REQUIRE(candidates != nullptr, FSA_E_ARG, "budgets need candidates");
    for (int i = 0; i < n_chunks; ++i)
      FSA_REQUIRE(candidates[i] >= 1, FSA_E_ARG, "candidates[%d]=%d must be >= 1", i,
                  candidates[i]);
  }
  const Schedule sc{n_chunks, cost, s_base, s_max};
  const double target = (1.0 - s_target) * total;
  const double r2 = std::sqrt(2.0), rn = std::sqrt((double)n_chunks);
  const double d = s_base - s_max;
  double lo = (d * r2 < d * rn ? d * r2 : d * rn) - 1.0;
  double hi = s_base * r2;
  if (s_base * rn > hi) hi = s_base * rn;
  if (0.0 > hi) hi = 0.0;
  hi = hi + 1.0;
  FSA_REQUIRE(!(sc.kept(lo) > target) && !(sc.kept(hi) < target), FSA_E_ARG,
              "the target sparsity %g cannot be reached with s_max %g", s_target, s_max);
  for (int it = 0; it < 200; ++it) {
    const double mid = lo + (hi - lo) * 0.5;
    if (mid <= lo || mid >= hi) break;
    if (sc.kept(mid) >= target)
      hi = mid;
    else
      lo = mid;
  }
  for (int i = 0; i < n_chunks; ++i) sparsity[i] = sc.sparsity(hi, i);
  if (budgets) {
    for (int i = 0; i < n_chunks; ++i) {
      const double k = std::floor((1.0 - sparsity[i]) * (double)candidates[i] + 0.5);
      const int c = candidates[i];
      budgets[i] = k < 1.0 ? 1 : (k > (double)c ? c : (int32_t)k);
    }
  }
  if (beta_out) *beta_out = hi;
  return FSA_OK;
}
