// ar_select.cpp -- host-side cost-guided protocol selector.
//
// "flash-comm: Self-Synchronizing Collective Communication for LLM
// Decoding", abstract: the readiness encoding is chosen by message size and
// the number of participating GPUs, trading synchronization overhead against
// the extra bytes an encoding moves.  "Why Microseconds Matter in AI
// Infrastructure", sections "What I learned from it" and "Where I think this
// is heading": the choice is made from measurements, with a performance model
// as the next step.  Here the model is the two-term latency/bandwidth form
// T_p(S) = alpha_p + beta_p * S per collective, protocol p, rank count and
// size range (the simulator kernels change regime with size, so one line per
// range; the committed table has a range per interval between measured
// sizes), fitted to measurements from this GPU by the Python side and
// passed in as a table.  Beyond the pages' protocol choice, the same model
// chooses between the one-shot and the two-shot all-reduce.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "../../include/ar.h"

static int select_in(const ar_cost_entry* table, int32_t nentries, int32_t collective,
                     int64_t payload_bytes, int32_t nranks, int32_t* proto_out,
                     double* predicted_us) {
  if (!table || nentries < 1 || !proto_out) return AR_EINVAL;
  if (payload_bytes < 0 || nranks < 1 || nranks > AR_MAX_RANKS) return AR_EINVAL;
  // rank count nearest to nranks among this collective's entries; ties go to
  // the smaller rank count
  int32_t n_use = -1;
  int best_dist = 0;
  for (int i = 0; i < nentries; ++i) {
    if (table[i].collective != collective) continue;
    const int dist = abs(table[i].nranks - nranks);
    if (n_use < 0 || dist < best_dist || (dist == best_dist && table[i].nranks < n_use)) {
      n_use = table[i].nranks;
      best_dist = dist;
    }
  }
  if (n_use < 0) return AR_EINVAL;
  // size range holding the payload: smallest upper end >= payload (no upper
  // end counts as infinite); if all end below it, the one ending last
  auto upper = [&](int i) {
    return table[i].max_bytes > 0 ? table[i].max_bytes : INT64_MAX;
  };
  int best = -1;
  int last = -1;
  for (int i = 0; i < nentries; ++i) {
    if (table[i].collective != collective || table[i].nranks != n_use) continue;
    const int64_t hi = upper(i);
    if (hi >= payload_bytes && (best < 0 || hi < upper(best))) best = i;
    if (last < 0 || hi > upper(last)) last = i;
  }
  if (best < 0) best = last;
  const ar_cost_entry& e = table[best];
  int choice = -1;
  double t_best = 0.0;
  for (int p = 0; p < 4; ++p) {
    const double a = e.alpha_us[p];
    const double b = e.beta_us_per_byte[p];
    if (!isfinite(a) || !isfinite(b)) continue;   // unavailable (NaN)
    const double t = a + b * (double)payload_bytes;
    if (choice < 0 || t < t_best) {   // strict: ties keep the lower id
      choice = p;
      t_best = t;
    }
  }
  if (choice < 0) return AR_EINVAL;
  *proto_out = choice;
  if (predicted_us) *predicted_us = t_best;
  return AR_OK;
}

extern "C" int ar_select_protocol(const ar_cost_entry* table, int32_t nentries,
                                  int64_t payload_bytes, int32_t nranks,
                                  int32_t* proto_out, double* predicted_us) {
  return select_in(table, nentries, AR_ALLREDUCE, payload_bytes, nranks, proto_out,
                   predicted_us);
}

extern "C" int ar_select_collective(const ar_cost_entry* table, int32_t nentries,
                                    int32_t collective, int64_t payload_bytes,
                                    int32_t nranks, int32_t* proto_out,
                                    double* predicted_us) {
  if (collective < AR_ALLREDUCE || collective > AR_TWOSHOT) return AR_EINVAL;
  return select_in(table, nentries, collective, payload_bytes, nranks, proto_out,
                   predicted_us);
}

extern "C" int ar_select_allreduce(const ar_cost_entry* table, int32_t nentries,
                                   int64_t payload_bytes, int32_t nranks,
                                   int32_t* collective_out, int32_t* proto_out,
                                   double* predicted_us) {
  if (!collective_out || !proto_out) return AR_EINVAL;
  int32_t p1 = -1;
  double t1 = 0.0;
  const int rc = select_in(table, nentries, AR_ALLREDUCE, payload_bytes, nranks, &p1, &t1);
  if (rc) return rc;
  int32_t p2 = -1;
  double t2 = 0.0;
  const bool two = select_in(table, nentries, AR_TWOSHOT, payload_bytes, nranks, &p2,
                             &t2) == AR_OK;
  if (two && t2 < t1) {
    *collective_out = AR_TWOSHOT;
    *proto_out = p2;
    if (predicted_us) *predicted_us = t2;
  } else {
    *collective_out = AR_ALLREDUCE;
    *proto_out = p1;
    if (predicted_us) *predicted_us = t1;
  }
  return AR_OK;
}
