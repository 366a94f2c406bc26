// Strict token-logprob kernels for gfx950 and the C-ABI declared in include/rlk_logp.h.
//
// Kernels:
//   k_full_g1     one workgroup (8 waves) per row: wave s summarises shard s,
//                 the summaries meet in LDS, thread 0 merges them and writes
//                 the reference logprob (the headline path, one launch).
//   k_summaries   groups > 1 or the support path: workgroup (row, g) runs the
//                 8/groups consecutive shards that a physical rank would own
//                 and stores their summaries in the workspace.
//   k_merge_full  one thread per row: the same merge as k_full_g1.
//   k_nucleus_g1  groups == 1 support path in one launch: one workgroup per
//                 row runs the 8 shard-waves, which also count every token
//                 into an LDS histogram of compressed BF16 ranks, merges the
//                 summaries (reference logprob), finds the top-k/top-p
//                 support from the exact integer histogram and writes the
//                 policy logprob.
//   k_nucleus     groups > 1: the same per-row support search on summaries
//                 that k_summaries stored in the workspace.
// Passages: RL-Kernel page "Configurable H100 consistency runs" (sampling,
// topology and mode/KL paragraphs; top-k independent of top-p in the command
// examples) and page "Reproduce and profile the Qwen3-8B TP4/CP2 experiment",
// section "How non-default CUDA topology reuses TP4/CP2" (per-virtual-shard
// summaries merged in fixed global-vocabulary order).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "logp_device.hpp"
#include "rlk_logp.h"
#include "support.hpp"

namespace rlk {

// Vectors per lane per chunk in the streaming loop.
constexpr int kChunk = 8;
constexpr int kRowThreads = kShards * kWave;  // 512

// Per-row, per-shard dispatch on the temperature (uniform across the workgroup).
template <typename Hook = NoHook>
__device__ __forceinline__ ShardSummary summarize_row_shard(const uint16_t* __restrict__ rowp, int shard,
                                                            int shard_width, int64_t vocab_real, float t,
                                                            Hook& hook) {
  ShardSummary s;
  s.r = 0.0f;
  s.l = 0.0f;
  s.m = -INFINITY;
  s.first = -1;
  if (!temperature_valid(t)) {
    s.l = NAN;
    return s;
  }
  const int64_t col0 = static_cast<int64_t>(shard) * shard_width;
  int64_t ncols64 = vocab_real - col0;
  ncols64 = ncols64 < 0 ? 0 : (ncols64 > shard_width ? shard_width : ncols64);
  const int ncols = static_cast<int>(ncols64);
  if (ncols == 0) return s;
  if (t == 0.0f) return summarize_shard_greedy(rowp, static_cast<int>(col0), ncols);
  const float c = kLog2e / t;  // IEEE float32 division
  return summarize_shard<kChunk>(rowp, static_cast<int>(col0), ncols, c, hook);
}

__device__ __forceinline__ float load_target_logit(const uint16_t* __restrict__ rowp, int64_t tg) {
  return __uint_as_float(static_cast<uint32_t>(rowp[tg]) << 16);
}

__global__ __launch_bounds__(kRowThreads) void k_full_g1(const uint16_t* __restrict__ logits, int64_t row_stride,
                                                         int shard_width, int64_t vocab_real,
                                                         const float* __restrict__ temperature,
                                                         const int64_t* __restrict__ target,
                                                         float* __restrict__ logp_out, float* __restrict__ lse_out) {
  __shared__ ShardSummary sm[kShards];
  const int64_t row = blockIdx.x;
  const int wave = threadIdx.x / kWave;
  const uint16_t* __restrict__ rowp = logits + row * row_stride;
  const float t = temperature[row];

  int64_t tg = -1;
  bool tok = false;
  float xt = 0.0f;
  if (threadIdx.x == 0) {
    tg = target[row];
    tok = (tg >= 0) && (tg < vocab_real);
    if (tok) xt = load_target_logit(rowp, tg);
  }
  NoHook none;
  const ShardSummary s = summarize_row_shard(rowp, wave, shard_width, vocab_real, t, none);
  if ((threadIdx.x & (kWave - 1)) == 0) sm[wave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const RowMerge mr = merge_row(sm, t, tok, tg, xt);
    logp_out[row] = mr.logp;
    if (lse_out) lse_out[row] = mr.lse;
  }
}

__global__ __launch_bounds__(kRowThreads) void k_summaries(const uint16_t* __restrict__ logits, int64_t row_stride,
                                                           int shard_width, int64_t vocab_real,
                                                           const float* __restrict__ temperature, int groups,
                                                           ShardSummary* __restrict__ ws) {
  const int waves_per_group = kShards / groups;
  const int64_t row = blockIdx.x / groups;
  const int g = blockIdx.x % groups;
  const int shard = g * waves_per_group + static_cast<int>(threadIdx.x / kWave);
  const uint16_t* __restrict__ rowp = logits + row * row_stride;
  const float t = temperature[row];
  NoHook none;
  const ShardSummary s = summarize_row_shard(rowp, shard, shard_width, vocab_real, t, none);
  if ((threadIdx.x & (kWave - 1)) == 0) ws[row * kShards + shard] = s;
}

__global__ __launch_bounds__(256) void k_merge_full(const uint16_t* __restrict__ logits, int64_t row_stride,
                                                    int64_t vocab_real, const float* __restrict__ temperature,
                                                    const int64_t* __restrict__ target,
                                                    const ShardSummary* __restrict__ ws, int64_t n_rows,
                                                    float* __restrict__ logp_out, float* __restrict__ lse_out) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (row >= n_rows) return;
  ShardSummary s[kShards];
#pragma unroll
  for (int k = 0; k < kShards; ++k) s[k] = ws[row * kShards + k];
  const float t = temperature[row];
  const int64_t tg = target[row];
  const bool tok = (tg >= 0) && (tg < vocab_real);
  const float xt = tok ? load_target_logit(logits + row * row_stride, tg) : 0.0f;
  const RowMerge mr = merge_row(s, t, tok, tg, xt);
  logp_out[row] = mr.logp;
  if (lse_out) lse_out[row] = mr.lse;
}

// ----------------------------------------------------------------------------
// Support path (top-k then top-p): see support.hpp.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kNucThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_nucleus_g1(const uint16_t* __restrict__ logits, int64_t row_stride,
                                                            int shard_width, int64_t vocab_real,
                                                            const float* __restrict__ temperature,
                                                            const float* __restrict__ top_p,
                                                            const int32_t* __restrict__ top_k,
                                                            const int64_t* __restrict__ target,
                                                            float* __restrict__ policy_out,
                                                            float* __restrict__ ref_out) {
  __shared__ NucLds L;
  const int64_t row = blockIdx.x;
  const int wave = threadIdx.x / kWave;
  const uint16_t* __restrict__ rowp = logits + row * row_stride;
  const float t = temperature[row];
  const float p = top_p[row];
  const int64_t k = top_k[row];
  if (search_needed(t, p, k, vocab_real)) {
    // the shard-waves build the key histogram while they stream the row
    window_clear(L);
    __syncthreads();
    WindowHook hook(L.u.win);
    const ShardSummary s = summarize_row_shard(rowp, wave, shard_width, vocab_real, t, hook);
    if ((threadIdx.x & (kWave - 1)) == 0) L.sm[wave] = s;
    hook.publish(L);
  } else {
    NoHook none;
    const ShardSummary s = summarize_row_shard(rowp, wave, shard_width, vocab_real, t, none);
    if ((threadIdx.x & (kWave - 1)) == 0) L.sm[wave] = s;
  }
  __syncthreads();
  nucleus_row(L, rowp, row, vocab_real, t, p, k, target[row], true, policy_out, ref_out);
}

__global__ __launch_bounds__(kNucThreads) void k_nucleus(const uint16_t* __restrict__ logits, int64_t row_stride,
                                                         int64_t vocab_real, const float* __restrict__ temperature,
                                                         const float* __restrict__ top_p,
                                                         const int32_t* __restrict__ top_k,
                                                         const int64_t* __restrict__ target,
                                                         const ShardSummary* __restrict__ ws,
                                                         float* __restrict__ policy_out, float* __restrict__ ref_out) {
  __shared__ NucLds L;
  const int64_t row = blockIdx.x;
  if (threadIdx.x < kShards) L.sm[threadIdx.x] = ws[row * kShards + threadIdx.x];
  __syncthreads();
  nucleus_row(L, logits + row * row_stride, row, vocab_real, temperature[row], top_p[row], top_k[row], target[row],
              false, policy_out, ref_out);
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
constexpr int64_t kMaxVocab = int64_t(1) << 30;

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static int32_t check_layout(int64_t n_rows, const rlk_vocab_layout* L) {
  if (L == nullptr) return RLK_ERR_NULL;
  if (n_rows < 0) return RLK_ERR_SHAPE;
  if (L->n_shards != kShards) return RLK_ERR_SHAPE;
  if (L->vocab_padded < 8 * kShards || L->vocab_padded > kMaxVocab) return RLK_ERR_SHAPE;
  if (L->vocab_padded % (8 * kShards) != 0) return RLK_ERR_SHAPE;
  if (L->vocab_real < 1 || L->vocab_real > L->vocab_padded) return RLK_ERR_SHAPE;
  if (L->row_stride < L->vocab_padded || L->row_stride % 8 != 0) return RLK_ERR_SHAPE;
  if (!(L->groups == 1 || L->groups == 2 || L->groups == 4 || L->groups == 8)) return RLK_ERR_GROUPS;
  if (n_rows > 0) {
    if (n_rows * static_cast<int64_t>(L->groups) > INT32_MAX) return RLK_ERR_SHAPE;
    if (L->row_stride > INT64_MAX / 2 / n_rows) return RLK_ERR_SHAPE;
  }
  return RLK_OK;
}

static size_t workspace_bytes(int64_t n_rows, const rlk_vocab_layout* L, bool /*nucleus*/) {
  if (L->groups == 1) return 0;
  return static_cast<size_t>(n_rows) * kShards * sizeof(ShardSummary);
}

static int32_t launched() { return hipGetLastError() == hipSuccess ? RLK_OK : RLK_ERR_HIP; }

}  // namespace rlk

extern "C" {

const char* rlk_status_string(int32_t status) {
  switch (status) {
    case RLK_OK: return "ok";
    case RLK_ERR_NULL: return "a required pointer is NULL";
    case RLK_ERR_ALIGN: return "misaligned pointer (logits and workspace need 16 bytes)";
    case RLK_ERR_SHAPE: return "n_rows or a layout field is out of range";
    case RLK_ERR_GROUPS: return "groups must be 1, 2, 4 or 8";
    case RLK_ERR_WORKSPACE: return "workspace missing or too small";
    case RLK_ERR_HIP: return "HIP runtime error while launching";
    default: return "unknown status";
  }
}

size_t rlk_logp_workspace_bytes(int64_t n_rows, const rlk_vocab_layout* layout, int32_t nucleus) {
  if (rlk::check_layout(n_rows, layout) != RLK_OK) return 0;
  return rlk::workspace_bytes(n_rows, layout, nucleus != 0);
}

int32_t rlk_logp_full(const uint16_t* logits, int64_t n_rows, const rlk_vocab_layout* layout,
                      const float* temperature, const int64_t* target, float* logp_out, float* lse_out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace rlk;
  int32_t st = check_layout(n_rows, layout);
  if (st != RLK_OK) return st;
  if (n_rows == 0) return RLK_OK;  // nothing to read or write: pointers may be NULL
  if (!logits || !temperature || !target || !logp_out) return RLK_ERR_NULL;
  if (!aligned(logits, 16) || !aligned(temperature, 4) || !aligned(target, 8) || !aligned(logp_out, 4) ||
      (lse_out && !aligned(lse_out, 4)))
    return RLK_ERR_ALIGN;
  const size_t need = rlk::workspace_bytes(n_rows, layout, false);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return RLK_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return RLK_ERR_ALIGN;
  }
  const int S = static_cast<int>(layout->vocab_padded / kShards);
  const int G = layout->groups;
  if (G == 1) {
    k_full_g1<<<dim3(static_cast<unsigned>(n_rows)), dim3(kRowThreads), 0, stream>>>(
        logits, layout->row_stride, S, layout->vocab_real, temperature, target, logp_out, lse_out);
    return launched();
  }
  ShardSummary* ws = static_cast<ShardSummary*>(workspace);
  k_summaries<<<dim3(static_cast<unsigned>(n_rows * G)), dim3(kShards / G * kWave), 0, stream>>>(
      logits, layout->row_stride, S, layout->vocab_real, temperature, G, ws);
  if ((st = launched()) != RLK_OK) return st;
  const unsigned blocks = static_cast<unsigned>((n_rows + 255) / 256);
  k_merge_full<<<dim3(blocks), dim3(256), 0, stream>>>(logits, layout->row_stride, layout->vocab_real,
                                                       temperature, target, ws, n_rows, logp_out, lse_out);
  return launched();
}

int32_t rlk_logp_nucleus(const uint16_t* logits, int64_t n_rows, const rlk_vocab_layout* layout,
                         const float* temperature, const float* top_p, const int32_t* top_k, const int64_t* target,
                         float* policy_out, float* ref_out, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  using namespace rlk;
  int32_t st = check_layout(n_rows, layout);
  if (st != RLK_OK) return st;
  if (n_rows == 0) return RLK_OK;  // nothing to read or write: pointers may be NULL
  if (!logits || !temperature || !top_p || !top_k || !target || !policy_out || !ref_out) return RLK_ERR_NULL;
  if (!aligned(logits, 16) || !aligned(temperature, 4) || !aligned(top_p, 4) || !aligned(top_k, 4) ||
      !aligned(target, 8) || !aligned(policy_out, 4) || !aligned(ref_out, 4))
    return RLK_ERR_ALIGN;
  const size_t need = rlk::workspace_bytes(n_rows, layout, true);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return RLK_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return RLK_ERR_ALIGN;
  }
  const int S = static_cast<int>(layout->vocab_padded / kShards);
  const int G = layout->groups;
  if (G == 1) {
    k_nucleus_g1<<<dim3(static_cast<unsigned>(n_rows)), dim3(kNucThreads), 0, stream>>>(
        logits, layout->row_stride, S, layout->vocab_real, temperature, top_p, top_k, target, policy_out, ref_out);
    return launched();
  }
  ShardSummary* ws = static_cast<ShardSummary*>(workspace);
  k_summaries<<<dim3(static_cast<unsigned>(n_rows * G)), dim3(kShards / G * kWave), 0, stream>>>(
      logits, layout->row_stride, S, layout->vocab_real, temperature, G, ws);
  if ((st = launched()) != RLK_OK) return st;
  k_nucleus<<<dim3(static_cast<unsigned>(n_rows)), dim3(kNucThreads), 0, stream>>>(
      logits, layout->row_stride, layout->vocab_real, temperature, top_p, top_k, target, ws, policy_out, ref_out);
  return launched();
}

}  // extern "C"
