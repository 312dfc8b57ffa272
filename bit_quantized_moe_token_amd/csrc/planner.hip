// Host-side planner of bit-plane releases (PagedWeight review page, "What
// carries the argument" and referee summary): a byte target becomes a
// sequence of one-plane bitwidth reductions chosen by predicted damage per
// released byte, damage d = max(eps, mu_i * g_i * eta_i).
#include "common.hpp"

MOEQ_API moeq_status moeq_plan_reductions(int32_t n, int32_t *q, const double *bytes, const double *g,
                                          const double *mu, const double *eta, double eps, double target,
                                          int32_t *order, int32_t max_actions, double *released,
                                          double *damage, int32_t *n_actions) {
  using namespace moeq;
  if (n < 0 || (n > 0 && (!q || !bytes || !g || !mu || !eta)) || !released || !damage || !n_actions)
    return fail(MOEQ_ERR_INVALID, "plan_reductions: null argument or n < 0");
  if (max_actions < 0 || (max_actions > 0 && !order))
    return fail(MOEQ_ERR_INVALID, "plan_reductions: order array missing");
  if (!(eps >= 0.0)) return fail(MOEQ_ERR_INVALID, "plan_reductions: eps must be >= 0");
  for (int i = 0; i < n; ++i) {
    if (q[i] < 2 || q[i] > 4) return fail(MOEQ_ERR_INVALID, "plan_reductions: q[%d]=%d not in 2..4", i, q[i]);
    for (int b = 1; b < 3; ++b)
      if (!(bytes[3 * i + b] > bytes[3 * i + b - 1]))
        return fail(MOEQ_ERR_INVALID, "plan_reductions: bytes of block %d must grow with q", i);
  }
  double rel = 0.0, dmg = 0.0;
  int na = 0;
  if (target > 0.0) {
    while (rel < target) {
      int best = -1;
      double best_key = 0.0, best_d = 0.0, best_r = 0.0;
      for (int i = 0; i < n; ++i) {
        if (q[i] <= 2) continue;
        const int qq = q[i];
        const double r = bytes[3 * i + qq - 2] - bytes[3 * i + qq - 3];
        const double prod = mu[i] * g[3 * i + qq - 3] * eta[i];
        const double d = prod > eps ? prod : eps;
        const double key = d / r;
        if (best < 0 || key < best_key) { best = i; best_key = key; best_d = d; best_r = r; }
      }
      if (best < 0) break;
      q[best] -= 1;
      if (na < max_actions) order[na] = best;
      ++na;
      rel += best_r;
      dmg += best_d;
    }
  }
  *released = rel;
  *damage = dmg;
  *n_actions = na;
  return MOEQ_OK;
}
