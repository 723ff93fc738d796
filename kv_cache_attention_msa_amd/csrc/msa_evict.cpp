// Eviction order of cached KV blocks (include/msa_evict.h).
//
// Score of block b at time t: c_b n_b min(1, lambda exp(-(t - t_b) / s)).
// Before its turning point (t - t_b <= s ln lambda) a block's score is
// c_b n_b, which does not change with time; past it the score is
// exp(ln(c_b n_b) + ln lambda + (t_b - t) / s), whose order among blocks does
// not change with time either (the exponential of Appendix A.1).  So the
// index keeps
//   * a min-heap of the blocks before their turning points, keyed c_b n_b;
//   * a min-heap of the blocks past them, keyed ln(c_b n_b) + (t_b - t0) / s
//     (t0 a fixed origin; lambda and t are common to all and left out);
//   * every block in a list by last access, oldest first.  The blocks past
//     their turning points are a prefix of that list; as time passes (or
//     lambda shrinks) its boundary moves forward and the blocks it passes
//     move from the first heap to the second, and back when lambda grows.
// Both heaps are indexed 4-ary heaps (each entry knows its position), so
// insert, touch, reposition, remove and evict are O(log n).
#include <cmath>
#include <limits>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "msa.h"
#include "msa_evict.h"

namespace msa {
int set_error_msg(int code, const std::string& msg);
}

namespace {

using msa::set_error_msg;

constexpr double kNegInf = -std::numeric_limits<double>::infinity();

struct Entry {
  int64_t id = 0;
  double cost = 0.0;    // c_b >= 0
  double n = 0.0;       // accesses
  double tb = 0.0;      // last access
  double lin = 0.0;     // c_b n_b: key before the turning point
  double lk = 0.0;      // ln(c_b n_b) + (t_b - t0) / s: key past it
  int32_t heap = -1;    // 0: before the turning point, 1: past it
  int32_t hpos = -1;
  int32_t prev = -1, next = -1;
};

}  // namespace

struct msa_evict {
  msa_latency_model model{};
  double s = 1.0, lam = 1.0, lnlam = 0.0, xstar = 0.0;   // turning point x* = s ln(lambda)
  double t0 = 0.0, last_now = kNegInf;
  bool have_t0 = false;
  std::vector<Entry> e;
  std::vector<int32_t> free_slots;
  std::unordered_map<int64_t, int32_t> where;
  std::vector<int32_t> h[2];
  int32_t head = -1, tail = -1;   // list by last access, oldest first
  int32_t first_flat = -1;        // first list entry before its turning point (-1: none)
};

namespace {

double key_of(const msa_evict* x, int32_t slot, int which) {
  return which == 0 ? x->e[slot].lin : x->e[slot].lk;
}

bool less(const msa_evict* x, int which, int32_t a, int32_t b) {
  const double ka = key_of(x, a, which), kb = key_of(x, b, which);
  return ka < kb || (ka == kb && x->e[a].id < x->e[b].id);
}

void place(msa_evict* x, int which, int32_t i, int32_t slot) {
  x->h[which][i] = slot;
  x->e[slot].hpos = i;
}

void sift_up(msa_evict* x, int which, int32_t i) {
  std::vector<int32_t>& h = x->h[which];
  const int32_t slot = h[i];
  while (i > 0) {
    const int32_t p = (i - 1) / 4;
    if (!less(x, which, slot, h[p])) break;
    place(x, which, i, h[p]);
    i = p;
  }
  place(x, which, i, slot);
}

void sift_down(msa_evict* x, int which, int32_t i) {
  std::vector<int32_t>& h = x->h[which];
  const int32_t n = (int32_t)h.size();
  const int32_t slot = h[i];
  for (;;) {
    const int32_t c0 = 4 * i + 1;
    if (c0 >= n) break;
    int32_t best = c0;
    for (int32_t c = c0 + 1; c < c0 + 4 && c < n; ++c)
      if (less(x, which, h[c], h[best])) best = c;
    if (!less(x, which, h[best], slot)) break;
    place(x, which, i, h[best]);
    i = best;
  }
  place(x, which, i, slot);
}

void heap_push(msa_evict* x, int which, int32_t slot) {
  x->e[slot].heap = which;
  x->h[which].push_back(slot);
  sift_up(x, which, (int32_t)x->h[which].size() - 1);
}

void heap_erase(msa_evict* x, int32_t slot) {
  const int which = x->e[slot].heap;
  std::vector<int32_t>& h = x->h[which];
  const int32_t i = x->e[slot].hpos;
  const int32_t last = h.back();
  h.pop_back();
  if (last != slot) {
    place(x, which, i, last);
    sift_up(x, which, i);
    sift_down(x, which, x->e[last].hpos);
  }
  x->e[slot].heap = -1;
  x->e[slot].hpos = -1;
}

void heap_fix(msa_evict* x, int32_t slot) {
  const int which = x->e[slot].heap;
  sift_up(x, which, x->e[slot].hpos);
  sift_down(x, which, x->e[slot].hpos);
}

void list_append(msa_evict* x, int32_t slot) {
  Entry& en = x->e[slot];
  en.prev = x->tail;
  en.next = -1;
  if (x->tail >= 0) x->e[x->tail].next = slot;
  else x->head = slot;
  x->tail = slot;
}

void list_unlink(msa_evict* x, int32_t slot) {
  Entry& en = x->e[slot];
  if (x->first_flat == slot) x->first_flat = en.next;
  if (en.prev >= 0) x->e[en.prev].next = en.next;
  else x->head = en.next;
  if (en.next >= 0) x->e[en.next].prev = en.prev;
  else x->tail = en.prev;
  en.prev = en.next = -1;
}

void set_keys(msa_evict* x, Entry& en) {
  const double cn = en.cost * en.n;
  en.lin = cn;
  en.lk = cn > 0.0 ? std::log(cn) + (en.tb - x->t0) / x->s : kNegInf;
}

bool before_turning_point(const msa_evict* x, const Entry& en, double now) { return now - en.tb <= x->xstar; }

// Move the blocks that passed their turning point by `now` to the second heap.
void advance(msa_evict* x, double now) {
  while (x->first_flat >= 0 && !before_turning_point(x, x->e[x->first_flat], now)) {
    const int32_t slot = x->first_flat;
    x->first_flat = x->e[slot].next;
    heap_erase(x, slot);
    heap_push(x, 1, slot);
  }
}

// After the turning point moved later: move blocks back to the first heap.
void retreat(msa_evict* x, double now) {
  int32_t slot = x->first_flat >= 0 ? x->e[x->first_flat].prev : x->tail;
  while (slot >= 0 && before_turning_point(x, x->e[slot], now)) {
    heap_erase(x, slot);
    heap_push(x, 0, slot);
    x->first_flat = slot;
    slot = x->e[slot].prev;
  }
}

// Append a block accessed at `now` at the list's tail, in the heap for its regime.
void enter(msa_evict* x, int32_t slot, double now) {
  list_append(x, slot);
  if (before_turning_point(x, x->e[slot], now)) {
    heap_push(x, 0, slot);
    if (x->first_flat < 0) x->first_flat = slot;
  } else {
    heap_push(x, 1, slot);   // lambda < 1: no block is ever before its turning point
  }
}

double direct_score(const msa_evict* x, const Entry& en, double now) {
  return en.cost * en.n * std::fmin(1.0, x->lam * std::exp(-(now - en.tb) / x->s));
}

double block_cost(const msa_evict* x, double l1, double q1) {
  const double* k = x->model.k;
  const double dt = k[4] * (l1 + 2.0 * q1) + (k[1] - k[2] + k[4]);   // Eq. 5
  return dt > 0.0 ? dt : 0.0;
}

int check_now(msa_evict* x, double now) {
  if (!std::isfinite(now)) return set_error_msg(MSA_ERR_INVALID_ARG, "time must be finite");
  if (now < x->last_now) return set_error_msg(MSA_ERR_INVALID_ARG, "time went back");
  x->last_now = now;
  if (!x->have_t0) {
    x->t0 = now;
    x->have_t0 = true;
  }
  return MSA_OK;
}

int find(const msa_evict* x, int64_t block, int32_t* slot) {
  auto it = x->where.find(block);
  if (it == x->where.end())
    return set_error_msg(MSA_ERR_INVALID_ARG, "block " + std::to_string(block) + " is not in the index");
  *slot = it->second;
  return MSA_OK;
}

bool good_pos(double l1, double q1) { return std::isfinite(l1) && std::isfinite(q1) && l1 >= 0.0 && q1 >= 0.0; }

void set_lambda_value(msa_evict* x, double lam) {
  x->lam = lam;
  x->lnlam = std::log(lam);
  x->xstar = x->s * x->lnlam;
}

}  // namespace

extern "C" {

int msa_evict_create(const msa_latency_model* model, double s, double lambda, msa_evict** out) {
  if (!model || !out) return set_error_msg(MSA_ERR_INVALID_ARG, "model or out is NULL");
  *out = nullptr;
  for (double k : model->k)
    if (!std::isfinite(k)) return set_error_msg(MSA_ERR_INVALID_ARG, "model coefficients must be finite");
  if (!(std::isfinite(s) && s > 0.0)) return set_error_msg(MSA_ERR_INVALID_ARG, "s must be finite and > 0");
  if (!(std::isfinite(lambda) && lambda > 0.0))
    return set_error_msg(MSA_ERR_INVALID_ARG, "lambda must be finite and > 0");
  msa_evict* x = new (std::nothrow) msa_evict();
  if (!x) return set_error_msg(MSA_ERR_OOM, "host allocation failed");
  x->model = *model;
  x->s = s;
  set_lambda_value(x, lambda);
  *out = x;
  return MSA_OK;
}

int msa_evict_destroy(msa_evict* idx) {
  delete idx;
  return MSA_OK;
}

int msa_evict_insert(msa_evict* x, int64_t block, double l1, double q1, double now) {
  if (!x) return set_error_msg(MSA_ERR_INVALID_ARG, "index is NULL");
  if (!good_pos(l1, q1)) return set_error_msg(MSA_ERR_INVALID_ARG, "l1 and q1 must be finite and >= 0");
  if (x->where.count(block)) return set_error_msg(MSA_ERR_INVALID_ARG, "block " + std::to_string(block) + " is already in the index");
  int rc = check_now(x, now);
  if (rc) return rc;
  advance(x, now);
  int32_t slot;
  try {
    if (!x->free_slots.empty()) {
      slot = x->free_slots.back();
      x->free_slots.pop_back();
    } else {
      slot = (int32_t)x->e.size();
      x->e.emplace_back();
    }
    x->where.emplace(block, slot);
    x->h[0].reserve(x->e.size());
    x->h[1].reserve(x->e.size());
  } catch (const std::bad_alloc&) {
    return set_error_msg(MSA_ERR_OOM, "host allocation failed");
  }
  Entry& en = x->e[slot];
  en = Entry{};
  en.id = block;
  en.cost = block_cost(x, l1, q1);
  en.n = 1.0;
  en.tb = now;
  set_keys(x, en);
  enter(x, slot, now);
  return MSA_OK;
}

int msa_evict_touch(msa_evict* x, int64_t block, double now) {
  if (!x) return set_error_msg(MSA_ERR_INVALID_ARG, "index is NULL");
  int32_t slot;
  int rc = find(x, block, &slot);
  if (rc) return rc;
  rc = check_now(x, now);
  if (rc) return rc;
  advance(x, now);
  list_unlink(x, slot);
  heap_erase(x, slot);
  Entry& en = x->e[slot];
  en.n += 1.0;
  en.tb = now;
  set_keys(x, en);
  enter(x, slot, now);
  return MSA_OK;
}

int msa_evict_set_position(msa_evict* x, int64_t block, double l1, double q1) {
  if (!x) return set_error_msg(MSA_ERR_INVALID_ARG, "index is NULL");
  if (!good_pos(l1, q1)) return set_error_msg(MSA_ERR_INVALID_ARG, "l1 and q1 must be finite and >= 0");
  int32_t slot;
  int rc = find(x, block, &slot);
  if (rc) return rc;
  Entry& en = x->e[slot];
  en.cost = block_cost(x, l1, q1);
  set_keys(x, en);
  heap_fix(x, slot);
  return MSA_OK;
}

int msa_evict_remove(msa_evict* x, int64_t block) {
  if (!x) return set_error_msg(MSA_ERR_INVALID_ARG, "index is NULL");
  int32_t slot;
  int rc = find(x, block, &slot);
  if (rc) return rc;
  list_unlink(x, slot);
  heap_erase(x, slot);
  x->where.erase(block);
  x->free_slots.push_back(slot);
  return MSA_OK;
}

int msa_evict_pop(msa_evict* x, double now, int64_t* block, double* score) {
  if (!x) return set_error_msg(MSA_ERR_INVALID_ARG, "index is NULL");
  if (x->where.empty()) return set_error_msg(MSA_ERR_INVALID_ARG, "the index is empty");
  int rc = check_now(x, now);
  if (rc) return rc;
  advance(x, now);
  // log scores of the two heaps' minima
  int32_t pick = -1;
  double best = 0.0;
  if (!x->h[0].empty()) {
    pick = x->h[0][0];
    best = x->e[pick].lin > 0.0 ? std::log(x->e[pick].lin) : kNegInf;
  }
  if (!x->h[1].empty()) {
    const int32_t c = x->h[1][0];
    const double ls = x->e[c].lk + x->lnlam - (now - x->t0) / x->s;
    if (pick < 0 || ls < best || (ls == best && x->e[c].id < x->e[pick].id)) {
      pick = c;
      best = ls;
    }
  }
  if (block) *block = x->e[pick].id;
  if (score) *score = direct_score(x, x->e[pick], now);
  return msa_evict_remove(x, x->e[pick].id);
}

int msa_evict_scan_min(msa_evict* x, double now, int64_t* block, double* score) {
  if (!x) return set_error_msg(MSA_ERR_INVALID_ARG, "index is NULL");
  if (x->where.empty()) return set_error_msg(MSA_ERR_INVALID_ARG, "the index is empty");
  int rc = check_now(x, now);
  if (rc) return rc;
  int32_t pick = -1;
  double best = 0.0;
  for (int32_t s = x->head; s >= 0; s = x->e[s].next) {
    const double sc = direct_score(x, x->e[s], now);
    if (pick < 0 || sc < best || (sc == best && x->e[s].id < x->e[pick].id)) {
      pick = s;
      best = sc;
    }
  }
  if (block) *block = x->e[pick].id;
  if (score) *score = best;
  return MSA_OK;
}

int msa_evict_score(msa_evict* x, int64_t block, double now, double* score) {
  if (!x || !score) return set_error_msg(MSA_ERR_INVALID_ARG, "index or score is NULL");
  if (!std::isfinite(now)) return set_error_msg(MSA_ERR_INVALID_ARG, "time must be finite");
  int32_t slot;
  int rc = find(x, block, &slot);
  if (rc) return rc;
  *score = direct_score(x, x->e[slot], now);
  return MSA_OK;
}

int msa_evict_set_lambda(msa_evict* x, double lambda, double now) {
  if (!x) return set_error_msg(MSA_ERR_INVALID_ARG, "index is NULL");
  if (!(std::isfinite(lambda) && lambda > 0.0))
    return set_error_msg(MSA_ERR_INVALID_ARG, "lambda must be finite and > 0");
  int rc = check_now(x, now);
  if (rc) return rc;
  advance(x, now);
  const double old = x->xstar;
  set_lambda_value(x, lambda);
  if (x->xstar < old) advance(x, now);
  else if (x->xstar > old) retreat(x, now);
  return MSA_OK;
}

int msa_evict_lambda_from_lifespan(double tau, double tau0, double alpha, double beta, double* lambda) {
  if (!lambda) return set_error_msg(MSA_ERR_INVALID_ARG, "lambda is NULL");
  if (!(std::isfinite(tau) && std::isfinite(tau0) && std::isfinite(alpha) && std::isfinite(beta) && alpha > 0.0 &&
        beta > 0.0))
    return set_error_msg(MSA_ERR_INVALID_ARG, "tau, tau0 must be finite; alpha, beta finite and > 0");
  const double l = std::exp((tau - tau0) / beta - tau / alpha);   // Eq. 10
  if (!(std::isfinite(l) && l > 0.0)) return set_error_msg(MSA_ERR_INVALID_ARG, "lambda out of range");
  *lambda = l;
  return MSA_OK;
}

int msa_evict_size(const msa_evict* x, int64_t* n) {
  if (!x || !n) return set_error_msg(MSA_ERR_INVALID_ARG, "NULL argument");
  *n = (int64_t)x->where.size();
  return MSA_OK;
}

}  // extern "C"
