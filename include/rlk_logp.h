/*
 * rlk_logp.h - strict, batch- and partition-invariant token log-probabilities
 * from BF16 logits, computed by HIP kernels for gfx950 (MI355X).
 *
 * Defining passages (RL-Kernel documentation pages):
 *  [CFG-SAMPLING] "Configurable H100 consistency runs", sampling paragraph:
 *      both sides scale the same BF16 model logits by a float32 temperature;
 *      temperature is finite and >= 0 (0 selects greedy sampling); top-p lies
 *      in (0, 1]; top-k is -1 (disabled) or a positive integer up to the real
 *      vocabulary size; the top-p/top-k support is computed over the real
 *      vocabulary; temperatures may differ per request.
 *  [CFG-TOPOLOGY] same page, topology paragraph: fixed virtual TP8 partitions
 *      and a padded vocabulary of 152576 across physical TP sizes.
 *  [CFG-KL] same page, mode/KL paragraph: the KL reference logprob is
 *      temperature-scaled over the full vocabulary; the policy logprob keeps
 *      its actual top-p/top-k support.
 *  [CFG-CMDS] same page, command examples: top-k is independent of top-p and
 *      temperature.
 *  [REPRO-CANON] "Reproduce and profile the Qwen3-8B TP4/CP2 experiment",
 *      section "How non-default CUDA topology reuses TP4/CP2": logp emits
 *      per-virtual-shard vocabulary summaries and merges them in fixed
 *      global-vocabulary order; a coarser physical rank owns several virtual
 *      shards, which only adds launches.
 *
 * What is computed, per row i (token position) with target column t_i:
 *   x_j   = BF16 logit of column j, widened exactly to float32, j < vocab_real
 *   z_j   = fl32(x_j / T_i)                       (IEEE division, [CFG-SAMPLING])
 *   lse_i = log(sum_j exp(z_j))                   (over the real vocabulary)
 *   ref_i = z_{t_i} - lse_i                       ([CFG-KL])
 * The sum is formed from 8 canonical shards of width vocab_padded/8; each
 * shard is reduced to a summary (an integer reference exponent r_s at or near
 * the shard maximum in log2 units, and l_s = sum of 2^(x_j*log2(e)/T - r_s)
 * accumulated in one fixed order), and the 8 summaries are merged left to
 * right as lse = ln2 * (R + log2(sum_s l_s * 2^(r_s - R))), R = max_s r_s
 * ([REPRO-CANON]). The order of every floating-point operation depends only
 * on the column geometry, never on the batch, the row position or `groups`,
 * so identical rows give identical output bytes in any call.
 *
 * Memory: every pointer argument is caller-owned DEVICE memory, except
 * `layout`, which is a host pointer read during the call. The library never
 * allocates, frees or synchronises: a call validates its arguments on the
 * host, enqueues kernels on `stream` and returns. Outputs are complete when
 * the stream reaches that point. Calls are hipGraph-capturable.
 *
 * Errors: argument errors detectable on the host return a negative status
 * before any HIP call is made (nothing is enqueued). A failed launch returns
 * RLK_ERR_HIP. Per-row values live on the device and are not checked on the
 * host; a row with an invalid temperature (NaN, +-inf, < 0) or target
 * (outside [0, vocab_real)), or whose real logits contain NaN or +inf, or are
 * all -inf, produces NaN outputs. Columns >= vocab_real are never used,
 * whatever they hold.
 */
#ifndef RLK_LOGP_H
#define RLK_LOGP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  RLK_OK = 0,
  RLK_ERR_NULL = -1,      /* a required pointer is NULL */
  RLK_ERR_ALIGN = -2,     /* logits/workspace not 16-byte aligned, or another array misaligned */
  RLK_ERR_SHAPE = -3,     /* n_rows (0 .. 2^22) or a layout field out of range */
  RLK_ERR_GROUPS = -4,    /* groups is not 1, 2, 4 or 8 */
  RLK_ERR_WORKSPACE = -5, /* workspace missing or smaller than rlk_logp_workspace_bytes() */
  RLK_ERR_HIP = -6,       /* the HIP runtime reported an error when launching */
  RLK_ERR_SCRATCH = -7    /* n_rows above RLK_NOALLOC_MAX_ROWS in rlk_logp_nucleus_noalloc */
};

/* Row layout of the logits [CFG-TOPOLOGY], [REPRO-CANON].
 * Row i starts at element i * row_stride of `logits`; columns are BF16 bit
 * patterns (uint16). The canonical partition splits columns [0, vocab_padded)
 * into n_shards shards of width vocab_padded / n_shards. */
typedef struct rlk_vocab_layout {
  int64_t vocab_padded; /* multiple of 8 * n_shards, 8 * n_shards <= vocab_padded <= 2^30 */
  int64_t vocab_real;   /* 1 <= vocab_real <= vocab_padded; columns >= vocab_real are ignored */
  int64_t row_stride;   /* elements between rows; >= vocab_padded and a multiple of 8 */
  int32_t n_shards;     /* canonical virtual shards; must be 8 */
  int32_t groups;       /* physical blocks per row (1, 2, 4 or 8): a block owns n_shards/groups
                           consecutive shards, like a physical TP rank owning several virtual
                           shards. Never changes any output byte. */
} rlk_vocab_layout;

/* Full-vocabulary (reference) logprob of target[i] for each row
 * [CFG-SAMPLING], [CFG-KL], [REPRO-CANON].
 *   logits       [n_rows * row_stride] BF16 bits, 16-byte aligned
 *   temperature  [n_rows] float32; 0 selects greedy: logp = 0 for the
 *                lowest-index maximum of the real logits, -inf elsewhere
 *   target       [n_rows] int64 column indices
 *   logp_out     [n_rows] float32
 *   lse_out      [n_rows] float32 log-sum-exp of the scaled row (NaN for
 *                greedy rows), or NULL
 *   workspace    rlk_logp_workspace_bytes(n_rows, layout, 0) bytes, 16-byte
 *                aligned; may be NULL when that size is 0 (groups == 1)
 * Returns RLK_OK or a negative status. n_rows == 0 (with a valid layout)
 * returns RLK_OK without reading any other argument and enqueues nothing. */
int32_t rlk_logp_full(const uint16_t* logits, int64_t n_rows, const rlk_vocab_layout* layout,
                      const float* temperature, const int64_t* target,
                      float* logp_out, float* lse_out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Per-row record of the support decision, written by rlk_logp_nucleus and read
 * by rlk_logp_backward [CFG-KL]. */
typedef struct rlk_support_state {
  float lse_support; /* log of the sum of exp(z_j) over the support (natural log);
                        equal to lse when the support is the whole real vocabulary;
                        NaN for greedy and invalid rows */
  float threshold;   /* smallest kept BF16 logit value: column j < vocab_real is in
                        the support iff x_j >= threshold; -inf when the support is
                        the whole real vocabulary */
  int32_t status;    /* 1: the target is in the support (policy logprob finite or
                        -inf only through a -inf target logit); 0: the target is
                        outside it (policy -inf); -1: no support (invalid top_p /
                        top_k, or a row maximum beyond the search's range; policy
                        NaN); -2: invalid row (reference NaN) */
  int32_t reserved;  /* 0 */
} rlk_support_state;

/* Policy logprob over the top-k-then-top-p support, and the full-vocabulary
 * reference logprob used for KL [CFG-SAMPLING], [CFG-KL], [CFG-CMDS].
 * Support of row i: top-k (when top_k[i] != -1 and < vocab_real) keeps every
 * column whose scaled logit is >= the k-th largest (ties at the boundary are
 * all kept); top-p (when top_p[i] < 1) then keeps, among those, every column
 * whose value is >= the largest value v for which the kept mass at values >= v
 * reaches top_p[i] times the mass of the top-k set.
 *   policy_out[i] = z_t - log(sum over the support of exp(z_j)) if t is in the
 *                   support, else -inf; exactly ref_out[i] when the support
 *                   is the whole real vocabulary; NaN for an invalid top_p
 *                   (outside (0, 1]) or top_k (not -1 and not in
 *                   [1, vocab_real]).
 *   ref_out[i]    = z_t - lse, the full-vocabulary logprob. For a row that
 *                   needs a support search (top_p < 1 or top_k < vocab_real,
 *                   T > 0) whose real tokens all lie in the search's window
 *                   (BF16 magnitudes in [2^-24, 4096), +-0, or -inf), with its
 *                   target among the real columns and its maximum in the
 *                   search's range (below), lse comes from the same exact
 *                   integer class masses as the policy: lse = (R +
 *                   log2(Z) - 40) * ln 2 with Z the row's total mass in units
 *                   of 2^(R-40); within the tolerance of rlk_logp_full's value
 *                   (a float32 ulp apart on the benchmark rows). Every other
 *                   row's reference is byte-identical to rlk_logp_full's
 *                   logp_out[i]. Either way the bytes depend only on the row.
 *   lse_out        [n_rows] float32, that lse (byte-identical to
 *                  rlk_logp_full's lse_out on the rows of its reference), or
 *                  NULL.
 *   support_out    [n_rows] rlk_support_state (16 bytes each), or NULL.
 *   top_p  [n_rows] float32;  top_k [n_rows] int32.
 *   workspace      rlk_logp_workspace_bytes(n_rows, layout, 1) bytes, 16-byte
 *                  aligned; may be NULL when that size is 0 (groups == 1).
 * Greedy rows (temperature 0) put a point mass on the lowest-index maximum for
 * both outputs. The support decision is taken on integer masses (64-bit, in
 * units of 2^-40 of the row's largest weight), so it is the same for any batch
 * or grouping; vocab_real must stay below 2^24 - 2^20 = 15728640 (else
 * RLK_ERR_SHAPE). A row whose largest scaled logit has |max x * log2(e) / T|
 * >= 2^20 (|x / T| above about 726817) gets no support: policy NaN and status
 * -1, the reference as usual. */
int32_t rlk_logp_nucleus(const uint16_t* logits, int64_t n_rows, const rlk_vocab_layout* layout,
                         const float* temperature, const float* top_p, const int32_t* top_k,
                         const int64_t* target, float* policy_out, float* ref_out,
                         float* lse_out, rlk_support_state* support_out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Rows that rlk_logp_nucleus_noalloc handles with groups > 1 (its static
 * scratch holds their shard summaries: 128 bytes per row, 4 MiB per GPU). */
#define RLK_NOALLOC_MAX_ROWS 32768

/* rlk_logp_nucleus without a workspace argument, for callers that cannot
 * allocate device memory (code under hipGraph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, outputs and bytes as
 * rlk_logp_nucleus; the caller still provides every input and output.
 * With groups > 1 the shard summaries go to a static device array of
 * RLK_NOALLOC_MAX_ROWS rows that the library keeps on each GPU it runs on
 * until the process ends (its address is looked up on the first call on a
 * device, with the current device; nothing is allocated). Every call on one
 * GPU shares that array, so calls that overlap on one GPU (concurrent streams
 * or host threads) race and must be serialised by the caller; a call writes
 * every summary it reads, so nothing needs clearing between calls.
 * Returns RLK_ERR_SCRATCH when groups > 1 and n_rows > RLK_NOALLOC_MAX_ROWS,
 * RLK_ERR_HIP when the scratch address cannot be obtained, otherwise what
 * rlk_logp_nucleus returns. With groups == 1 no scratch is used. */
int32_t rlk_logp_nucleus_noalloc(const uint16_t* logits, int64_t n_rows, const rlk_vocab_layout* layout,
                                 const float* temperature, const float* top_p, const int32_t* top_k,
                                 const int64_t* target, float* policy_out, float* ref_out,
                                 float* lse_out, rlk_support_state* support_out, hipStream_t stream);

/* Gradient of sum_i (grad_ref[i] * ref_i + grad_policy[i] * policy_i) with
 * respect to the BF16 logits, as BF16 (round to nearest even), for training
 * on these logprobs (page "H100 canonical CP backward validation", Change
 * section: the training step back-propagates through the logprob; [CFG-KL]
 * for the two terms). For a row with temperature T > 0 and target t:
 *   d/dx_j = ( [j == t] * (g_r + g_p) - g_r * p_j - g_p * [x_j >= thr] * q_j ) / T
 * with p_j = exp(z_j - lse), q_j = exp(z_j - lse_support), g_r = grad_ref[i],
 * g_p = grad_policy[i] when the target is in the support (status 1) and 0
 * when it is outside (the policy logprob is the constant -inf there). The
 * support is piecewise constant in the logits and contributes no term. The
 * target column is formed as (g_r * -expm1(ref) + g_p * -expm1(policy)) / T,
 * which keeps 1 - p_t accurate when p_t is near 1.
 *   logits        as for the forward call that produced the row statistics
 *   temperature, target  as for the forward call
 *   ref_logp, lse [n_rows] float32: logp_out and lse_out of rlk_logp_full
 *                 (or ref_out and lse_out of rlk_logp_nucleus) on these rows
 *   grad_ref      [n_rows] float32 upstream gradient of ref_i, or NULL (no
 *                 reference term; ref_logp and lse may then be NULL)
 *   policy_logp, support  [n_rows] policy_out and support_out of
 *                 rlk_logp_nucleus on these rows
 *   grad_policy   [n_rows] float32 upstream gradient of policy_i, or NULL (no
 *                 policy term; policy_logp and support may then be NULL)
 *   grad_logits   [n_rows * grad_stride] BF16 bits, 16-byte aligned; columns
 *                 [0, vocab_padded) of each row are written (pad columns get
 *                 0), columns beyond are left untouched
 *   grad_stride   >= vocab_padded and a multiple of 8
 * Row rules, in order: both upstream gradients 0 -> zeros; an invalid row
 * (invalid temperature or target, ref NaN, or status -2) -> NaN on the real
 * columns; T == 0 (greedy: piecewise-constant logprob) -> zeros; a nonzero
 * grad_policy with status -1 -> NaN on the real columns. The pad columns are
 * always 0. Each output depends only on its own row's inputs, so the bytes do
 * not change with the batch or `groups` (which is not used here).
 * At least one of grad_ref / grad_policy must be given (else RLK_ERR_NULL).
 * Returns RLK_OK or a negative status; n_rows == 0 enqueues nothing. */
int32_t rlk_logp_backward(const uint16_t* logits, int64_t n_rows, const rlk_vocab_layout* layout,
                          const float* temperature, const int64_t* target,
                          const float* ref_logp, const float* lse, const float* grad_ref,
                          const float* policy_logp, const rlk_support_state* support, const float* grad_policy,
                          uint16_t* grad_logits, int64_t grad_stride, hipStream_t stream);

/* Vocabulary-parallel form [REPRO-CANON], [CFG-TOPOLOGY]: with `groups` = G
 * ranks, rank r holds the columns [r*C, (r+1)*C) of every row, C = 8/G shards
 * of width vocab_padded/8 (the canonical partition does not depend on G).
 *
 * rlk_logp_shard_summaries: rank `rank` reduces its slice to its 8/G shard
 * summaries.
 *   logits_slice  [n_rows * slice_stride] BF16 bits, 16-byte aligned; row i's
 *                 column r*C + j is logits_slice[i * slice_stride + j]
 *   slice_stride  >= C and a multiple of 8
 *   temperature, target  as for rlk_logp_full (target is a global column)
 *   summaries_out rlk_logp_summary_bytes(n_rows, layout) bytes, 16-byte
 *                 aligned: n_rows * (8/G) records of 16 bytes, record
 *                 (i, j) at index i * (8/G) + j for local shard j. A record is
 *                 {float r; float l; float m; int32 aux}: for a row with
 *                 T > 0, l = sum of 2^(x*log2(e)/T - r) over the shard's real
 *                 columns in a fixed order, r an integer-valued reference
 *                 exponent, aux = the target's BF16 bits if the target column
 *                 lies in this shard, else -1; for T == 0, m = the shard's
 *                 maximum and aux = its lowest global column.
 *   layout->row_stride is not used (it must still be valid).
 * rlk_logp_merge: given every rank's summaries concatenated in rank order
 * (what an all-gather of summaries_out produces: rank r's block at offset
 * r * rlk_logp_summary_bytes(); summaries_bytes >= n_rows * 128), merges each
 * row's 8 summaries left to right and writes the same logp_out / lse_out
 * bytes as rlk_logp_full on the whole rows, for every G.
 * Both return RLK_OK or a negative status (rank outside [0, G) or a bad
 * slice_stride is RLK_ERR_SHAPE; a short summary buffer RLK_ERR_WORKSPACE);
 * n_rows == 0 enqueues nothing. */
int32_t rlk_logp_shard_summaries(const uint16_t* logits_slice, int64_t n_rows, const rlk_vocab_layout* layout,
                                 int32_t rank, int64_t slice_stride, const float* temperature,
                                 const int64_t* target, void* summaries_out, size_t summaries_bytes,
                                 hipStream_t stream);

int32_t rlk_logp_merge(const void* summaries, size_t summaries_bytes, int64_t n_rows,
                       const rlk_vocab_layout* layout, const float* temperature, const int64_t* target,
                       float* logp_out, float* lse_out, hipStream_t stream);

/* Bytes of one rank's summaries: n_rows * (8/groups) * 16. 0 for an invalid
 * layout or n_rows < 0. */
size_t rlk_logp_summary_bytes(int64_t n_rows, const rlk_vocab_layout* layout);

/* Bytes of device workspace rlk_logp_full / rlk_logp_nucleus need: 0 when
 * groups == 1, else n_rows * 128 (8 shard summaries of 16 bytes per row), for
 * either entry point. Returns 0 for an invalid layout or n_rows < 0. */
size_t rlk_logp_workspace_bytes(int64_t n_rows, const rlk_vocab_layout* layout, int32_t nucleus);

/* Static, NUL-terminated description of a status code. */
const char* rlk_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* RLK_LOGP_H */
