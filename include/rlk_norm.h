/*
 * rlk_norm.h - order-independent L2 norm of FP32 gradients on gfx950
 * (MI355X): the sum of the FP32 squares is accumulated in integer exponent
 * bins, so the result does not depend on the order of the elements, on how
 * they are split into tensors, launches or ranks, or on the schedule of any
 * atomic operation.
 *
 * Defining passage: RL-Kernel page "H100 canonical CP backward validation",
 * Change section: the training step's L2 norm of the gradients sums the FP32
 * squares in integer exponent bins before the distributed reduction, and that
 * norm drives gradient clipping; Timing and scope section: a 10M-element
 * BF16-derived FP32 norm microbenchmark.
 *
 * What is computed for float32 values x_i:
 *   s_i   = fl32(x_i * x_i)                 (IEEE float32 multiply, nearest even)
 *   bins  : integer words with sum_e bin[e] * 2^(max(e, 1) - 150) = S, the
 *           exact sum of the finite squares. A square s_i = m_i *
 *           2^(max(e, 1) - 150) (m_i its 24-bit integer significand, hidden
 *           bit included for e >= 1) adds m_i to bin[e]; squares of nearby
 *           exponents may first be summed exactly in fixed point and added as
 *           two 32-bit halves to bins lo and lo + 32 - the same value. How the
 *           value is spread over the words depends on the launch, never the
 *           value. NaN squares are counted in n_nan, +inf squares (overflow,
 *           infinite x) in n_inf.
 *   sumsq = fl64(S) (nearest even); NaN if n_nan > 0, else +inf if n_inf > 0
 *   norm  = fl32(sqrt(sumsq))
 * Bins of several calls, tensors or ranks add as integers: a distributed
 * reduction is an integer all-reduce (sum) of the rlk_norm_bins words, after
 * which every rank finalises to the same bytes.
 *
 * Memory: every pointer is caller-owned DEVICE memory; nothing is allocated,
 * freed or synchronised. Argument errors detectable on the host return a
 * negative status (codes of rlk_logp.h) before any HIP call.
 */
#ifndef RLK_NORM_H
#define RLK_NORM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "rlk_logp.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Integer accumulator of the squares (2112 bytes, 8-byte aligned). bin[255]
 * is never used by a finite square and stays 0. The word-by-word integer sum of two
 * accumulators is the accumulator of the union of their values. The total
 * number of accumulated values must stay below 2^39 (no word can overflow). */
typedef struct rlk_norm_bins {
  uint64_t bin[256];
  uint64_t n_nan;
  uint64_t n_inf;
  uint64_t reserved[6]; /* 0 */
} rlk_norm_bins;

/* Sets every word of *bins to 0 (a kernel, so it may be captured in a graph). */
int32_t rlk_l2norm_zero(rlk_norm_bins* bins, hipStream_t stream);

/* Adds the squares of x[0 .. n) to *bins.
 *   x     float32 values, 4-byte aligned (any offset into a buffer)
 *   n     0 <= n < 2^39; n == 0 enqueues nothing and reads no pointer
 * Several calls on the same bins (one per gradient tensor, in any order, on
 * any streams once ordered before the finalisation) give the bins of the
 * concatenation. */
int32_t rlk_l2norm_accumulate(const float* x, int64_t n, rlk_norm_bins* bins, hipStream_t stream);

/* sumsq_out[0] = fl64 of the exact sum, norm_out[0] = fl32(sqrt(sumsq)), from
 * *bins (which are not modified). Either output may be NULL, not both. */
int32_t rlk_l2norm_finalize(const rlk_norm_bins* bins, double* sumsq_out, float* norm_out, hipStream_t stream);

/* accumulate + finalize of one array (two launches). *workspace must be
 * all-zero on entry (rlk_l2norm_zero once before the first call); the
 * finalisation clears it again, so consecutive calls on one stream need no
 * clearing. Calls that overlap on one workspace race. n == 0 gives 0. */
int32_t rlk_l2norm(const float* x, int64_t n, rlk_norm_bins* workspace, double* sumsq_out, float* norm_out,
                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RLK_NORM_H */
