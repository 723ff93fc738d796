/*
 * msa_latency.h -- the Eq. 5 latency model of the AsymCache / Multi-Segment
 * Attention paper (Figure 6 caption), fitted to this library's own timings.
 * Part of libmsa.so; host only (no HIP call), thread-safe.
 *
 * A request's context is four regions in position order: l1 cached blocks, q1
 * blocks recomputed this step, l2 cached blocks and q2 new blocks.  The pages
 * print only the marginal cost of recomputing one more block instead of
 * keeping it cached,
 *   dT_B = T(l1, q1 + 1, l2 - 1, q2) - T(l1, q1, l2, q2) = k5 (l1 + 2 q1) + (k2 - k3 + k5),
 * with hardware-dependent coefficients.  This library takes the plainest T
 * whose difference is exactly that:
 *   T = k1 + k2 (q1 + q2) + k3 (l1 + l2) + k4 q2 (l1 + q1 + l2 + q2) + k5 q1 (l1 + q1)
 * (fixed cost; per computed block; per cached block read; new blocks attending
 * to the whole context; recomputed blocks attending to the prefix and to
 * themselves).  Region sizes are in blocks of MSA_BLOCK_SIZE tokens.
 *
 * Return values as in msa.h (MSA_OK or MSA_ERR_INVALID_ARG, message in
 * msa_last_error()).
 */
#ifndef MSA_LATENCY_H_
#define MSA_LATENCY_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  double k[5];       /* k1..k5, in the time unit of the samples (per block, per block^2) */
  double rms;        /* root-mean-square residual of the fit (relative to T if `relative`) */
  int32_t n;         /* samples used                                                    */
  int32_t relative;  /* 1: residuals were taken relative to the measured time           */
} msa_latency_model;

/* Least-squares fit of k1..k5 to n samples, each five doubles
 * (l1, q1, l2, q2, T) in host memory: minimises the sum of squared residuals
 * T_model - T, each divided by T when relative != 0 (then every T must be > 0).
 * Needs n >= 5 samples that determine all five coefficients (for instance
 * some with q1 > 0 and some with q2 > 0 at several context sizes); region
 * sizes must be >= 0 and everything finite.  Errors: INVALID_ARG (bad
 * arguments, or samples that leave a coefficient undetermined). */
int msa_latency_fit(const double* samples, int32_t n, int32_t relative, msa_latency_model* out);

/* T(l1, q1, l2, q2) of a fitted model. */
int msa_latency_eval(const msa_latency_model* model, double l1, double q1, double l2, double q2, double* t);

/* Eq. 5: dT_B at (l1, q1) of a fitted model. */
int msa_latency_delta_b(const msa_latency_model* model, double l1, double q1, double* dt);

/* Adaptive chunk size (the pages' adaptive chunking scheduler, abstract and
 * summary: chunk sizes chosen for hardware utilisation).  For the next step of
 * a request whose context holds l1 cached, q1 recomputed and l2 cached blocks
 * and which still has `remaining` >= 1 new blocks to prefill: the largest c in
 * [1, remaining] whose predicted step time T(l1, q1, l2, c) is <= budget (the
 * step-time bound that keeps co-scheduled decode steps on time), so each step
 * does as much work as the bound allows; 1 if even one block exceeds it.
 * Errors: INVALID_ARG (NULL pointers, remaining < 1, non-finite arguments). */
int msa_chunk_blocks(const msa_latency_model* model, double l1, double q1, double l2, int32_t remaining,
                     double budget, int32_t* chunk);

#ifdef __cplusplus
}
#endif

#endif /* MSA_LATENCY_H_ */
