// Predicted-KL step control on the host: the annealed budget and the closed
// form shrink factor that keep the predicted policy change of a step within
// it ("LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
// Sketches", paragraph "Step control."; the walk-through page on LoGRA,
// section "Predicted-KL Step Control"). The readings (isotropic Fisher
// phi I, one factor per step, linear anneal) and the contract are stated
// with the declarations in include/logra.h. Host arithmetic only, in double.
#include <math.h>

#include "../../include/logra.h"

namespace {

bool finite_nonneg(double x) { return isfinite(x) && x >= 0.0; }

}  // namespace

extern "C" {

double logra_kl_budget_at(const logra_kl_budget *b, uint64_t step) {
    if (!b || !finite_nonneg(b->delta_start) || !finite_nonneg(b->delta_end)) return NAN;
    if (b->anneal_steps == 0 || step >= b->anneal_steps) return b->delta_end;
    const double frac = static_cast<double>(step) / static_cast<double>(b->anneal_steps);
    return b->delta_start + (b->delta_end - b->delta_start) * frac;
}

logra_status logra_kl_step_scale(const float *sqnorm, int64_t n, float lr, double fisher_scale,
                                 double delta, float *scales, double *kl_pred, double *kl_after) {
    if (n < 0 || !kl_pred || (n > 0 && (!sqnorm || !scales))) return LOGRA_ERR_INVALID_ARGUMENT;
    if (!isfinite(lr) || !isfinite(fisher_scale) || !(fisher_scale > 0.0) || !finite_nonneg(delta))
        return LOGRA_ERR_INVALID_ARGUMENT;
    // predicted KL of the unscaled update: 0.5 phi lr^2 sum of the kept sqnorms
    double sum = 0.0;
    for (int64_t m = 0; m < n; ++m) {
        const double q = sqnorm[m];
        if (finite_nonneg(q)) sum += q;
    }
    const double lr2 = static_cast<double>(lr) * static_cast<double>(lr);
    const double kl = 0.5 * fisher_scale * lr2 * sum;
    // quadratic model: KL(gamma dW) = gamma^2 KL(dW)
    const double gamma = kl <= delta ? 1.0 : sqrt(delta / kl);
    for (int64_t m = 0; m < n; ++m) scales[m] = finite_nonneg(sqnorm[m]) ? static_cast<float>(gamma) : 0.f;
    *kl_pred = kl;
    if (kl_after) *kl_after = gamma * gamma * kl;
    return LOGRA_OK;
}

}  // extern "C"
