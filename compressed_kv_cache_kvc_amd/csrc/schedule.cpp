// Per-layer keep budgets: the pyramid schedules of the pages, host side.
//
// Two schedules of the fraction r_l of a base budget that layer l (of n)
// keeps, with opposite directions on the pages:
//  * linear ("KV Cache optimization techniques" tutorial, section 2.3,
//    PyramidKV): r_l = 1 - 0.8 * (l / n), everything at the first layer down
//    to 0.2 + 0.8 / n at the last (shallow layers keep more);
//  * quadratic (eviction-and-reuse survey, section 4, the eviction engine's
//    pyramid ratio): r_l = r + (1 - r) * (l / n)^2 from a base ratio r, growing
//    with depth. The page fixes n = 80 as an assumption; here n is the
//    caller's layer count.
// budget_l = (int)(base * r_l), truncated toward zero as the pages' int()
// does, then raised to min_budget (the sinks and recent window must fit).
// Arithmetic in double, in the pages' order, so the integers are exact
// functions of the inputs.
#include <stdint.h>

#include "kvc.h"

namespace kvc {
int32_t fail(int32_t status, const char* fmt, ...);
void clear_error();
}  // namespace kvc

extern "C" int32_t kvc_layer_budgets(int32_t schedule, int32_t num_layers, int32_t base, double base_ratio,
                                     int32_t min_budget, int32_t* budgets_host) {
  kvc::clear_error();
  if (!budgets_host) return kvc::fail(KVC_ERR_INVALID_ARG, "budgets_host must not be NULL");
  if (num_layers < 1 || base < 1 || min_budget < 0)
    return kvc::fail(KVC_ERR_INVALID_ARG, "need num_layers >= 1, base >= 1 and min_budget >= 0");
  if (schedule != KVC_SCHEDULE_LINEAR && schedule != KVC_SCHEDULE_QUADRATIC)
    return kvc::fail(KVC_ERR_INVALID_ARG, "unknown schedule %d", schedule);
  if (schedule == KVC_SCHEDULE_QUADRATIC && !(base_ratio >= 0.0 && base_ratio <= 1.0))
    return kvc::fail(KVC_ERR_INVALID_ARG, "base_ratio must lie in [0, 1]");
  for (int32_t l = 0; l < num_layers; ++l) {
    const double x = (double)l / (double)num_layers;
    const double r = schedule == KVC_SCHEDULE_LINEAR ? 1.0 - 0.8 * x : base_ratio + (1.0 - base_ratio) * (x * x);
    const int32_t b = (int32_t)((double)base * r);
    budgets_host[l] = b < min_budget ? min_budget : b;
  }
  return KVC_OK;
}
