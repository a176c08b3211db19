// Host side of the per-layer readiness gate and the landmark-count rule
// ("Flux2TTRTrainer", section "How the distillation works": fail-closed
// readiness from enough updates and a low EMA cosine distance, with
// hysteresis; section "Inputs worth setting": landmark fraction/min/max and a
// readiness threshold). Plain host code: no GPU calls.
#include <cmath>

#include "validate.hpp"

extern "C" {

ttr_status ttr_gate_update(const ttr_gate_config* cfg, ttr_gate_state* st, double distance) {
  if (cfg == nullptr || st == nullptr) return TTR_ERR_NULL;
  if (!(cfg->ema_rate >= 0.0 && cfg->ema_rate < 1.0) || !(cfg->threshold_on >= 0.0) ||
      !(cfg->threshold_off >= cfg->threshold_on) || cfg->min_updates < 0)
    return TTR_ERR_SHAPE;
  if (!std::isfinite(distance)) {  // fail closed: an unusable measurement withdraws the student
    st->ready = 0;
    return TTR_ERR_SHAPE;
  }
  st->ema = st->updates == 0 ? distance : cfg->ema_rate * st->ema + (1.0 - cfg->ema_rate) * distance;
  st->updates += 1;
  if (st->ready) {
    if (st->ema > cfg->threshold_off) st->ready = 0;
  } else if (st->updates >= cfg->min_updates && st->ema <= cfg->threshold_on) {
    st->ready = 1;
  }
  return TTR_OK;
}

int32_t ttr_landmark_count(int32_t N, double fraction, int32_t lmin, int32_t lmax) {
  if (N < 0 || !(fraction >= 0.0) || lmin < 0 || lmax < lmin) return -1;
  const double r = std::floor(fraction * (double)N + 0.5);
  int64_t L = r > 2147483647.0 ? 2147483647 : (int64_t)r;
  if (L > lmax) L = lmax;
  if (L < lmin) L = lmin;
  if (L > N) L = N;
  return (int32_t)L;
}

}  // extern "C"
