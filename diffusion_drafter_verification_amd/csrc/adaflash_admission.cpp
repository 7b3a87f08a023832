// Verification-batch admission controller (host side).
//
// AdaFlash review (ZH), section 2.3, and AdaFlash review (EN), "Adaptive
// request scheduling for variable verification lengths": the verify batch is
// packed to sum_i k_hat_i tokens, so the number of requests a round can take
// varies; the scheduler keeps an exponential moving average of the requests a
// round actually advanced, N_hat <- (1 - beta) N_hat + beta N, admits up to
// that many, and sends requests that still overflow the budget back to the
// pending queue.
//
// Per round: propose() = the running requests, then pending ones in arrival
// order until the batch holds max(1, floor(N_hat + 0.5)); commit(k_hat)
// removes the most recently placed requests while sum k_hat exceeds the
// token budget (keeping at least one), puts them back at the front of the
// pending queue in their order, sets N = the batch size and updates N_hat;
// finish(ids) drops the requests that completed.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_set>
#include <vector>

#include "../../include/adaflash.h"

namespace {

struct Admission {
  double beta = 0.5;
  double n_hat = 0.0;
  int64_t budget = 1;
  std::deque<int64_t> pending;
  std::vector<int64_t> active;

  int target() const {
    const double t = std::floor(n_hat + 0.5);
    return t < 1.0 ? 1 : (t > 1e9 ? 1000000000 : (int)t);
  }
};

}  // namespace

extern "C" {

void* adaflash_admission_create(double beta, double n_hat0, int64_t budget_tokens) {
  if (!(beta > 0.0 && beta <= 1.0) || !(n_hat0 >= 0.0) || std::isinf(n_hat0) || budget_tokens < 1) return nullptr;
  Admission* a = new (std::nothrow) Admission();
  if (!a) return nullptr;
  a->beta = beta;
  a->n_hat = n_hat0;
  a->budget = budget_tokens;
  return a;
}

void adaflash_admission_destroy(void* h) { delete static_cast<Admission*>(h); }

int adaflash_admission_enqueue(void* h, const int64_t* ids, int n) {
  if (!h || n < 0 || (n > 0 && !ids)) return ADAFLASH_E_INVALID;
  Admission* a = static_cast<Admission*>(h);
  for (int i = 0; i < n; ++i) a->pending.push_back(ids[i]);
  return ADAFLASH_OK;
}

int adaflash_admission_propose(void* h, int64_t* out_ids, int cap) {
  if (!h || cap < 0 || (cap > 0 && !out_ids)) return ADAFLASH_E_INVALID;
  Admission* a = static_cast<Admission*>(h);
  const size_t t = (size_t)a->target();
  // How many the batch will hold: check the caller's capacity first, so that
  // a rejected call changes nothing.
  size_t want = a->active.size();
  if (want < t) want += std::min(t - want, a->pending.size());
  if (want > (size_t)cap) return ADAFLASH_E_INVALID;
  while (a->active.size() < t && !a->pending.empty()) {
    a->active.push_back(a->pending.front());
    a->pending.pop_front();
  }
  for (size_t i = 0; i < a->active.size(); ++i) out_ids[i] = a->active[i];
  return (int)a->active.size();
}

int adaflash_admission_commit(void* h, const int32_t* k_hat, int n, int64_t* out_ids) {
  if (!h || n < 0 || (n > 0 && (!k_hat || !out_ids))) return ADAFLASH_E_INVALID;
  Admission* a = static_cast<Admission*>(h);
  if ((size_t)n != a->active.size()) return ADAFLASH_E_INVALID;
  int64_t total = 0;
  for (int i = 0; i < n; ++i) total += k_hat[i];
  int keep = n;
  while (total > a->budget && keep > 1) {
    --keep;
    total -= k_hat[keep];
  }
  // Overflow back to the front of the pending queue, order kept.
  for (int i = n - 1; i >= keep; --i) a->pending.push_front(a->active[i]);
  a->active.resize(keep);
  // (two products and a sum, each rounded: no fused multiply-add)
  const double kept = (1.0 - a->beta) * a->n_hat;
  const double seen = a->beta * (double)keep;
  a->n_hat = kept + seen;
  for (int i = 0; i < keep; ++i) out_ids[i] = a->active[i];
  return keep;
}

int adaflash_admission_finish(void* h, const int64_t* done_ids, int n) {
  if (!h || n < 0 || (n > 0 && !done_ids)) return ADAFLASH_E_INVALID;
  Admission* a = static_cast<Admission*>(h);
  std::unordered_set<int64_t> done(done_ids, done_ids + n);
  std::vector<int64_t> keep;
  keep.reserve(a->active.size());
  for (int64_t r : a->active)
    if (!done.count(r)) keep.push_back(r);
  a->active.swap(keep);
  return ADAFLASH_OK;
}

double adaflash_admission_estimate(const void* h) { return h ? static_cast<const Admission*>(h)->n_hat : NAN; }

int adaflash_admission_pending(const void* h) {
  return h ? (int)static_cast<const Admission*>(h)->pending.size() : ADAFLASH_E_INVALID;
}

}  // extern "C"
