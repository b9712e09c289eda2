// Host-side scheduling pieces of the packed verification batch, after "AdaFlash: Adaptive Speculative
// Decoding with Online Self-Improvement for High-Concurrency LLM Inference" (besthub.dev article),
// section "Infrastructure: Async Training & Variable-Length Batching": requests with different
// predicted verification lengths are packed into compact batches, and an exponential moving average
// of the capacity sets the next round's budget. The packed layout (offsets, lengths) is what the
// verify / fused entry points take.

#include <cmath>
#include <cstdint>

#include "opd_internal.h"

namespace {

opd_status_t pfail(opd_status_t s, const char* msg) { return opd::record_error(s, msg); }

}  // namespace

extern "C" {

opd_status_t opd_capacity_init(opd_capacity_t* c, double beta) {
  if (!c) return pfail(OPD_ERR_NULL, "capacity state must be non-NULL");
  if (!(beta >= 0.0 && beta <= 1.0)) return pfail(OPD_ERR_PARAM, "beta must lie in [0, 1]");
  c->ema = 0.0;
  c->beta = beta;
  c->n_obs = 0;
  return OPD_OK;
}

opd_status_t opd_capacity_observe(opd_capacity_t* c, double observed_rows, int64_t* budget_rows) {
  if (!c || !budget_rows) return pfail(OPD_ERR_NULL, "capacity state and budget must be non-NULL");
  if (!(observed_rows >= 0.0) || std::isinf(observed_rows))
    return pfail(OPD_ERR_PARAM, "observed capacity must be finite and >= 0");
  // the first observation initialises the estimate; later ones are blended with weight 1 - beta
  c->ema = c->n_obs == 0 ? observed_rows : c->beta * c->ema + (1.0 - c->beta) * observed_rows;
  if (c->n_obs < INT32_MAX) ++c->n_obs;
  *budget_rows = static_cast<int64_t>(std::floor(c->ema));
  return OPD_OK;
}

opd_status_t opd_pack_first_fit(const int32_t* lengths, int32_t n_pending, int64_t budget_rows,
                                int32_t max_requests, int32_t* selected, int32_t* offsets,
                                int32_t* packed_lengths, int32_t* n_selected, int64_t* n_rows) {
  if (n_pending < 0 || budget_rows < 0 || max_requests < 0)
    return pfail(OPD_ERR_SHAPE, "n_pending, budget_rows and max_requests must be >= 0");
  if (!offsets || !n_selected || !n_rows) return pfail(OPD_ERR_NULL, "offsets, n_selected, n_rows must be non-NULL");
  if (n_pending > 0 && (!lengths || !selected || !packed_lengths))
    return pfail(OPD_ERR_NULL, "lengths, selected and packed_lengths must be non-NULL");
  for (int32_t r = 0; r < n_pending; ++r) {
    if (lengths[r] < 1) return pfail(OPD_ERR_PARAM, "predicted lengths must be >= 1");
  }
  int32_t n = 0;
  int64_t used = 0;
  offsets[0] = 0;
  for (int32_t r = 0; r < n_pending; ++r) {
    if (max_requests > 0 && n == max_requests) break;
    if (used + lengths[r] <= budget_rows) {  // first fit, arrival order: later requests may still fit
      selected[n] = r;
      packed_lengths[n] = lengths[r];
      used += lengths[r];
      ++n;
      offsets[n] = static_cast<int32_t>(used);
    }
  }
  *n_selected = n;
  *n_rows = used;
  return OPD_OK;
}

}  // extern "C"
