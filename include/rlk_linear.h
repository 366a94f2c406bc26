/*
 * rlk_linear.h - the LM-head linear layer and the fused "linear-logp" on
 * gfx950 (MI355X): BF16 hidden states times the BF16 vocabulary projection
 * with MFMA matrix instructions, and the strict token logprob computed from
 * those logits without writing them to memory.
 *
 * Defining passages (RL-Kernel documentation pages):
 *  [LINEAR-LOGP] "Reproduce and profile the Qwen3-8B TP4/CP2 experiment",
 *      section "Capture logs, status, and validation evidence": the run log
 *      is audited for `linear-logp` among the logprob backend markers (the
 *      LM-head linear fused with the logprob).
 *  [CFG-SAMPLING], [CFG-KL], [REPRO-CANON] as in rlk_logp.h: BF16 model
 *      logits, float32 temperature scaling, full-vocabulary reference
 *      logprob, summaries merged in a fixed global vocabulary order.
 *
 * What is computed, for row i (a token position) and vocabulary entry j:
 *   acc_ij = sum_k h_ik * w_jk     (float32 accumulation on the matrix cores;
 *                                    the order over k depends only on k)
 *   x_ij   = bf16(acc_ij)          (round to nearest even: the model's BF16
 *                                    logits)
 * rlk_linear writes x (pad columns j >= vocab_real as BF16 -inf).
 * rlk_linear_logp computes, from the same x_ij, the reference logprob of
 * target[i] exactly as rlk_logp.h defines it (temperature, greedy rows,
 * invalid rows), except that the row's log-sum-exp is merged from summaries
 * of 128-column tiles (in tile order) instead of the 8 canonical shards. The
 * tile grid does not depend on the batch (and its tiles nest in the canonical
 * shards of the 152576-column vocabulary), so identical rows give identical
 * bytes in any batch; the value agrees with rlk_logp_full on rlk_linear's
 * output to within float32 rounding of the sums.
 *
 * Shapes: hidden [n_rows x d_model] (row stride hidden_stride), weight
 * [vocab_real x d_model] (row stride weight_stride; rows >= vocab_real are
 * never read), both BF16 bit patterns, 16-byte aligned, strides multiples of
 * 8 and at most 2^21; d_model a multiple of 64 in [64, 65536]. layout->row_stride is the row
 * stride of rlk_linear's output (and is only validated by rlk_linear_logp);
 * layout->groups is validated; only the vocabulary-parallel entry points below use it.
 *
 * Memory: every pointer is caller-owned DEVICE memory except `layout` (host);
 * nothing is allocated, freed or synchronised. Argument errors detectable on
 * the host return a negative status (codes of rlk_logp.h) before any HIP
 * call; n_rows == 0 enqueues nothing.
 */
#ifndef RLK_LINEAR_H
#define RLK_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "rlk_logp.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Logits x = bf16(hidden . weight^T) into logits_out [n_rows x layout->row_stride]:
 * columns [0, vocab_real) hold x, [vocab_real, vocab_padded) BF16 -inf, the
 * rest of each row is not written. */
int32_t rlk_linear(const uint16_t* hidden, int64_t n_rows, int64_t d_model, int64_t hidden_stride,
                   const uint16_t* weight, int64_t weight_stride, const rlk_vocab_layout* layout,
                   uint16_t* logits_out, hipStream_t stream);

/* Reference logprob of target[i] under the temperature-scaled softmax of row
 * i of bf16(hidden . weight^T) over the real vocabulary, without writing the
 * logits [LINEAR-LOGP], [CFG-SAMPLING], [CFG-KL].
 *   temperature [n_rows] float32 (0: greedy), target [n_rows] int64
 *   logp_out [n_rows] float32; lse_out [n_rows] float32 or NULL
 *   workspace rlk_linear_logp_workspace_bytes(n_rows, layout) bytes, 16-byte
 *             aligned (one 16-byte summary per row and 128-column tile). */
int32_t rlk_linear_logp(const uint16_t* hidden, int64_t n_rows, int64_t d_model, int64_t hidden_stride,
                        const uint16_t* weight, int64_t weight_stride, const rlk_vocab_layout* layout,
                        const float* temperature, const int64_t* target, float* logp_out, float* lse_out,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* n_rows * ceil(vocab_padded / 128) * 16 bytes; 0 for an invalid layout or n_rows < 0. */
size_t rlk_linear_logp_workspace_bytes(int64_t n_rows, const rlk_vocab_layout* layout);

/* Vocabulary-parallel form [REPRO-CANON]: with G = layout->groups ranks, rank
 * r holds the projection rows of columns [r*C, (r+1)*C), C = vocab_padded / G
 * (a multiple of 128), and the same hidden states.
 * rlk_linear_logp_summaries: rank `rank` reduces its columns to n_rows * C/128
 * summaries of 128 columns (16 bytes each, record (i, j) at i * C/128 + j,
 * the target's BF16 logit carried by the summary holding the target column).
 *   weight_shard  the rank's projection rows: row j is vocabulary entry
 *                 r*C + j, for the min(C, vocab_real - r*C) entries below
 *                 vocab_real (none when r*C >= vocab_real; the pointer must
 *                 still be valid and aligned)
 *   summaries_out rlk_linear_logp_summary_bytes(n_rows, layout) bytes
 * rlk_linear_logp_merge: from every rank's summaries concatenated in rank
 * order (what an all-gather yields), the same logp_out / lse_out bytes as
 * rlk_linear_logp on the whole projection, for every G.
 * A C that is not a multiple of 128 or a rank outside [0, G) is
 * RLK_ERR_SHAPE; a short buffer RLK_ERR_WORKSPACE. */
int32_t rlk_linear_logp_summaries(const uint16_t* hidden, int64_t n_rows, int64_t d_model, int64_t hidden_stride,
                                  const uint16_t* weight_shard, int64_t weight_stride, const rlk_vocab_layout* layout,
                                  int32_t rank, const float* temperature, const int64_t* target,
                                  void* summaries_out, size_t summaries_bytes, hipStream_t stream);

int32_t rlk_linear_logp_merge(const void* summaries, size_t summaries_bytes, int64_t n_rows,
                              const rlk_vocab_layout* layout, const float* temperature, const int64_t* target,
                              float* logp_out, float* lse_out, hipStream_t stream);

/* One rank's summary bytes: n_rows * (vocab_padded / groups / 128) * 16; 0 for
 * an invalid layout, n_rows < 0 or a per-rank width that is not a multiple of 128. */
size_t rlk_linear_logp_summary_bytes(int64_t n_rows, const rlk_vocab_layout* layout);

#ifdef __cplusplus
}
#endif

#endif /* RLK_LINEAR_H */
