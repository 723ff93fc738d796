/*
 * msa_evict.h -- computation-latency-aware eviction order of cached KV blocks,
 * the cache eviction policy of the AsymCache / Multi-Segment Attention paper:
 * keep the blocks whose loss would cost the most, weighing how often they are
 * hit against what recomputing them costs the attention kernel (abstract;
 * Figure 6 caption, Eq. 5; Figure 8 caption and Figure 9's axes; Figure 10
 * caption, Eq. 10; Appendix A.1).  Part of libmsa.so; host only (no HIP
 * call).  An index is not thread-safe: one thread at a time per index.
 *
 * Score of a cached block b at time t (the lowest score is evicted first):
 *
 *   score_b(t) = c_b * n_b * w(t - t_b),   w(x) = min(1, lambda * exp(-x / s))
 *
 *   c_b  recomputation cost: dT_B of a fitted latency model (Eq. 5,
 *        k5 (l1 + 2 q1) + (k2 - k3 + k5)) at the block's place in its request,
 *        l1 cached and q1 recomputed blocks before it; a negative value counts
 *        as 0 (such a block is evicted first);
 *   n_b  accesses so far (the insertion and every hit since): frequency;
 *   t_b  time of the last access;
 *   w    the piecewise exponential weight (Figure 8): full weight until the
 *        turning point x* = s ln(lambda), exponential decay with time scale s
 *        after it.  lambda rescales the decaying part, which is the same as
 *        moving the turning point (Figure 10 caption); it may be set directly
 *        or from the average block lifespan by Eq. 10 (msa_evict_lambda_from_
 *        lifespan).  With lambda <= 1 every block is past its turning point.
 *
 * The pages give the score's ingredients and Eq. 10 but their text is cut off
 * before the formula that combines them; the form above is this library's
 * reading.  What fixes its shape is the order-preserving rule of Appendix
 * A.1 (only an exponential decay leaves the relative order of blocks that are
 * not accessed unchanged as time passes): past the turning point, the scores
 * of all blocks shrink by the same factor, so an ordering keyed once, at the
 * last access, stays valid, and the index keeps two heaps (blocks before and
 * past their turning points) and a list of blocks by last access: insert,
 * touch, reposition, remove and evict cost O(log n), against O(n) for a
 * rescoring scan (Figure 9: eviction time against 4-10 x 10^3 cached blocks).
 *
 * Times are doubles in any unit (s in the same unit); the `now` of successive
 * calls on one index must not decrease.  Ties are broken by the smaller
 * block id.  Return values as in msa.h (MSA_OK, MSA_ERR_INVALID_ARG,
 * MSA_ERR_OOM; message in msa_last_error()).
 */
#ifndef MSA_EVICT_H_
#define MSA_EVICT_H_

#include <stdint.h>

#include "msa_latency.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct msa_evict msa_evict;

/* New, empty index whose costs come from `model` (copied) with decay time
 * scale s > 0 and lambda > 0, both finite.  Errors: INVALID_ARG, OOM. */
int msa_evict_create(const msa_latency_model* model, double s, double lambda, msa_evict** out);

/* Free an index (NULL accepted). */
int msa_evict_destroy(msa_evict* idx);

/* Cache block `block` (any id not in the index) at time `now`: one access,
 * cost dT_B(l1, q1) with l1, q1 >= 0 finite.  Errors: INVALID_ARG (id
 * present, bad numbers, time going back), OOM. */
int msa_evict_insert(msa_evict* idx, int64_t block, double l1, double q1, double now);

/* A hit on `block` at time `now`: one more access, last access now.
 * Errors: INVALID_ARG (id absent, time going back). */
int msa_evict_touch(msa_evict* idx, int64_t block, double now);

/* The block's place in its request changed (blocks before it cached or
 * evicted): its cost becomes dT_B(l1, q1).  Errors: INVALID_ARG. */
int msa_evict_set_position(msa_evict* idx, int64_t block, double l1, double q1);

/* Drop `block` from the index without evicting it by score (for instance its
 * request ended).  Errors: INVALID_ARG (id absent). */
int msa_evict_remove(msa_evict* idx, int64_t block);

/* Evict: remove the block of lowest score at time `now`, returned in *block
 * with its score in *score (either may be NULL).  Errors: INVALID_ARG (empty
 * index, time going back). */
int msa_evict_pop(msa_evict* idx, double now, int64_t* block, double* score);

/* The block `pop` would evict at `now` and its score, found by rescoring
 * every block (O(n)); the index is not changed.  A reference for the heap
 * order and the O(n) baseline of the eviction-time comparison.
 * Errors: INVALID_ARG (empty index, time going back). */
int msa_evict_scan_min(msa_evict* idx, double now, int64_t* block, double* score);

/* Score of `block` at time `now`.  Errors: INVALID_ARG. */
int msa_evict_score(msa_evict* idx, int64_t block, double now, double* score);

/* Set lambda (> 0, finite) at time `now`; blocks cross between the two heaps
 * as the turning point moves.  Errors: INVALID_ARG. */
int msa_evict_set_lambda(msa_evict* idx, double lambda, double now);

/* Eq. 10: lambda = exp((tau - tau0) / beta - tau / alpha) for the average
 * block lifespan tau seen over a sliding window and constants tau0, alpha,
 * beta (alpha, beta > 0).  Errors: INVALID_ARG (non-finite arguments or
 * result). */
int msa_evict_lambda_from_lifespan(double tau, double tau0, double alpha, double beta, double* lambda);

/* Number of blocks in the index. */
int msa_evict_size(const msa_evict* idx, int64_t* n);

#ifdef __cplusplus
}
#endif

#endif /* MSA_EVICT_H_ */
