// Strict token-logprob kernels for gfx950 and the C-ABI declared in include/rlk_logp.h.
//
// Kernels:
//   k_full_g1          one workgroup (8 waves) per row: wave s summarises
//                      shard s, the summaries meet in LDS, thread 0 merges
//                      them and writes the reference logprob (one launch).
//   k_rank_summaries   workgroup (row, rank) runs the 8/groups consecutive
//                      shard-waves a rank of a vocabulary-parallel layout owns
//                      and stores their 16-byte summaries rank-major; used by
//                      groups > 1 and by rlk_logp_shard_summaries on a slice.
//   k_merge            one thread per row: the same fixed-order merge over the
//                      rank-major summaries (groups > 1, rlk_logp_merge).
//   k_nucleus_g1       the support path: a row that needs a search is
//                      streamed once by the shard-waves, which only count its
//                      tokens into an LDS window of BF16 classes; the eight
//                      waves then sum the exact integer class masses step by
//                      step, and wave 0 takes the reference logprob, the
//                      top-k/top-p support and the policy logprob from them
//                      (a second pass for the float32 shard summaries on the
//                      rare searched rows that cannot use the window). Rows
//                      without a search stream the float32 shard summaries
//                      (groups == 1) or read those k_rank_summaries stored
//                      for them (groups > 1).
//   k_backward         gradient of the reference and policy logprobs with
//                      respect to the BF16 logits, from the forward's per-row
//                      statistics; 1024-thread workgroups over (row, column
//                      chunk) items in row-major order (backward.hpp).
// Passages: RL-Kernel page "Configurable H100 consistency runs" (sampling,
// topology and mode/KL paragraphs; top-k independent of top-p in the command
// examples) and page "Reproduce and profile the Qwen3-8B TP4/CP2 experiment",
// section "How non-default CUDA topology reuses TP4/CP2" (per-virtual-shard
// summaries merged in fixed global-vocabulary order; a coarser physical rank
// owns several virtual shards).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "backward.hpp"
#include "logp_device.hpp"
#include "rlk_logp.h"
#include "support.hpp"

namespace rlk {

// Vectors per lane per chunk in the streaming loop (kRefGroup under a hook
// that widens late: those kernels run more waves per SIMD).
constexpr int kChunk = 8;
constexpr int kRowThreads = kShards * kWave;  // 512

// Summary of the shard whose first column (global index col0) is at `shard`,
// for a row with temperature t and target column tg. Uniform across the wave;
// dispatches on the temperature (uniform across the workgroup).
template <typename Hook = NoHook>
__device__ __forceinline__ ShardSummary summarize_row_shard(const uint16_t* __restrict__ shard, int64_t col0,
                                                            int shard_width, int64_t vocab_real, float t,
                                                            int64_t tg, Hook& hook) {
  ShardSummary s;
  s.r = 0.0f;
  s.l = 0.0f;
  s.m = -INFINITY;
  s.aux = -1;
  if (!temperature_valid(t)) {
    s.l = NAN;
    return s;
  }
  int64_t ncols64 = vocab_real - col0;
  ncols64 = ncols64 < 0 ? 0 : (ncols64 > shard_width ? shard_width : ncols64);
  const int ncols = static_cast<int>(ncols64);
  if (ncols == 0) return s;
  if (t == 0.0f) return summarize_shard_greedy(shard, static_cast<int>(col0), ncols);
  const float c = kLog2e / t;  // IEEE float32 division
  s = summarize_shard<(Hook::kLateWiden ? kRefGroup : kChunk)>(shard, ncols, c, hook);
  if (tg >= col0 && tg < col0 + ncols) s.aux = static_cast<int32_t>(shard[tg - col0]);
  return s;
}

__global__ __launch_bounds__(kRowThreads) void k_full_g1(const uint16_t* __restrict__ logits, int64_t row_stride,
                                                         int shard_width, int64_t vocab_real,
                                                         const float* __restrict__ temperature,
                                                         const int64_t* __restrict__ target,
                                                         float* __restrict__ logp_out, float* __restrict__ lse_out) {
  __shared__ ShardSummary sm[kShards];
  const int64_t row = blockIdx.x;
  const int wave = threadIdx.x / kWave;
  const int64_t col0 = static_cast<int64_t>(wave) * shard_width;
  const uint16_t* __restrict__ rowp = logits + row * row_stride;
  const float t = temperature[row];
  const int64_t tg = target[row];
  NoHook none;
  const ShardSummary s = summarize_row_shard(rowp + col0, col0, shard_width, vocab_real, t, tg, none);
  if ((threadIdx.x & (kWave - 1)) == 0) sm[wave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const bool tok = (tg >= 0) && (tg < vocab_real);
    const RowMerge mr = merge_row(sm, t, tok, tg, shard_width);
    logp_out[row] = mr.logp;
    if (lse_out) lse_out[row] = mr.lse;
  }
}

// Workgroup b handles row b / ranks_in_grid and rank rank0 + b % ranks_in_grid,
// whose slice of the row starts at base + (b % ranks_in_grid) * rank_col_step +
// row * slice_stride and holds shards [rank * spr, rank * spr + spr) (spr =
// 8 / groups = waves per workgroup). Writes out[((b % ranks_in_grid) * n_rows +
// row) * spr + wave]. With the support parameters (top_p non-null), rows that
// need a support search are skipped: the support kernel takes their
// reference from the exact class masses, or streams their summaries itself.
__global__ __launch_bounds__(kRowThreads) void k_rank_summaries(const uint16_t* __restrict__ base,
                                                                int64_t slice_stride, int64_t rank_col_step,
                                                                int rank0, int ranks_in_grid, int spr,
                                                                int shard_width, int64_t vocab_real, int64_t n_rows,
                                                                const float* __restrict__ temperature,
                                                                const int64_t* __restrict__ target,
                                                                const float* __restrict__ top_p,
                                                                const int32_t* __restrict__ top_k,
                                                                ShardSummary* __restrict__ out) {
  const int64_t row = blockIdx.x / ranks_in_grid;
  if (top_p != nullptr && search_needed(temperature[row], top_p[row], top_k[row], vocab_real)) return;
  const int rr = static_cast<int>(blockIdx.x % ranks_in_grid);
  const int wave = static_cast<int>(threadIdx.x / kWave);
  const int shard = (rank0 + rr) * spr + wave;
  const int64_t col0 = static_cast<int64_t>(shard) * shard_width;
  const uint16_t* __restrict__ sp =
      base + rr * rank_col_step + row * slice_stride + static_cast<int64_t>(wave) * shard_width;
  NoHook none;
  const ShardSummary s = summarize_row_shard(sp, col0, shard_width, vocab_real, temperature[row], target[row], none);
  if ((threadIdx.x & (kWave - 1)) == 0) out[(static_cast<int64_t>(rr) * n_rows + row) * spr + wave] = s;
}

// Loads the 8 summaries of a row from the rank-major layout.
__device__ __forceinline__ void load_row_summaries(const ShardSummary* __restrict__ ws, int64_t row, int64_t n_rows,
                                                   int spr, ShardSummary* s) {
#pragma unroll
  for (int k = 0; k < kShards; ++k) s[k] = ws[(static_cast<int64_t>(k / spr) * n_rows + row) * spr + (k % spr)];
}

__global__ __launch_bounds__(256) void k_merge(const ShardSummary* __restrict__ ws, int64_t n_rows, int spr,
                                               int shard_width, int64_t vocab_real,
                                               const float* __restrict__ temperature,
                                               const int64_t* __restrict__ target, float* __restrict__ logp_out,
                                               float* __restrict__ lse_out) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (row >= n_rows) return;
  ShardSummary s[kShards];
  load_row_summaries(ws, row, n_rows, spr, s);
  const int64_t tg = target[row];
  const bool tok = (tg >= 0) && (tg < vocab_real);
  const RowMerge mr = merge_row(s, temperature[row], tok, tg, shard_width);
  logp_out[row] = mr.logp;
  if (lse_out) lse_out[row] = mr.lse;
}

// ----------------------------------------------------------------------------
// Support path (top-k then top-p): see support.hpp.
// ----------------------------------------------------------------------------
// kStored == false (groups == 1): a row without a search streams its float32
// shard summaries here. kStored == true (groups > 1): k_rank_summaries stored
// them, split over `groups` workgroups per row, rank-major in ws (spr = 8 /
// groups summaries per rank); a row with a search is handled the same way in
// both, from one pass that counts its tokens.
template <bool kStored>
__global__ __launch_bounds__(kNucThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void k_nucleus_g1(
    const uint16_t* __restrict__ logits, int64_t row_stride, int shard_width, int64_t vocab_real,
    const float* __restrict__ temperature, const float* __restrict__ top_p, const int32_t* __restrict__ top_k,
    const int64_t* __restrict__ target, float* __restrict__ policy_out, float* __restrict__ ref_out,
    float* __restrict__ lse_out, rlk_support_state* __restrict__ state_out, const ShardSummary* __restrict__ ws,
    int64_t n_rows, int spr) {
  __shared__ NucLds L;
  const int64_t row = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform: offsets in SGPRs
  const int64_t col0 = static_cast<int64_t>(wave) * shard_width;
  const uint16_t* __restrict__ rowp = logits + row * row_stride;
  const float t = temperature[row];
  const float p = top_p[row];
  const int64_t k = top_k[row];
  const int64_t tg = target[row];
  if (!search_needed(t, p, k, vocab_real)) {
    // the reference from the shard summaries; the policy is the reference or NaN
    if constexpr (kStored) {
      if (threadIdx.x < kShards) {
        const int sh = threadIdx.x;
        L.sm[sh] = ws[(static_cast<int64_t>(sh / spr) * n_rows + row) * spr + (sh % spr)];
      }
    } else {
      NoHookLate none;
      const ShardSummary s = summarize_row_shard(rowp + col0, col0, shard_width, vocab_real, t, tg, none);
      if ((threadIdx.x & (kWave - 1)) == 0) L.sm[wave] = s;
    }
    __syncthreads();
    if (wave == 0) unsearched_row(L, row, vocab_real, shard_width, t, p, k, tg, policy_out, ref_out, lse_out, state_out);
    return;
  }
  // The shard-waves only count the row's tokens into the window; the wavefront
  // whose shard holds the target reads its BF16 pattern.
  window_clear(L);
  __syncthreads();
  {
    int64_t nc = vocab_real - col0;
    nc = nc < 0 ? 0 : (nc > shard_width ? shard_width : nc);
    const bool own_target = (tg >= col0) && (tg < col0 + nc);  // wave-uniform
    const uint32_t tb = own_target ? static_cast<uint32_t>(rowp[tg]) : 0u;  // issued before the pass
    WindowHook hook(L.u.win);
    count_shard<kRefGroup>(rowp + col0, static_cast<int>(nc), static_cast<int>(threadIdx.x & (kWave - 1)), hook);
    hook.publish(L);
    if (own_target && (threadIdx.x & (kWave - 1)) == 0) L.tbits = tb;
  }
  __syncthreads();
  bool odd = false;  // block-uniform: a real token outside the window
  for (int w = 0; w < kNucWaves; ++w) odd |= (L.red_flag[w] != 0);
  if (!odd && exact_row(L, row, vocab_real, t, p, k, tg, L.tbits, policy_out, ref_out, lse_out, state_out)) return;
  // The other rows (a token outside the window, no finite token, a target
  // outside the real columns, a maximum beyond the search's range): the
  // float32 shard summaries from a second pass, then the block-wide driver.
  {
    NoHookLate none;
    const ShardSummary s = summarize_row_shard(rowp + col0, col0, shard_width, vocab_real, t, tg, none);
    if ((threadIdx.x & (kWave - 1)) == 0) L.sm[wave] = s;
  }
  __syncthreads();
  nucleus_row(L, rowp, row, vocab_real, shard_width, t, p, k, tg, policy_out, ref_out, lse_out, state_out);
}

// ----------------------------------------------------------------------------
// Backward: see backward.hpp. Row rules in order: both upstream gradients 0
// -> zeros; invalid row -> NaN (real columns); greedy -> zeros; a policy
// gradient with invalid top-p/top-k -> NaN; else the gradient.
// ----------------------------------------------------------------------------
// Per-row set-up of the gradient; returns 0 to compute, 1 for zeros, 2 for NaN.
__device__ __forceinline__ int backward_row(int64_t row, int64_t vocab_real, const float* __restrict__ temperature,
                                            const int64_t* __restrict__ target, const float* __restrict__ ref_logp,
                                            const float* __restrict__ lse, const float* __restrict__ grad_ref,
                                            const float* __restrict__ policy_logp,
                                            const rlk_support_state* __restrict__ support,
                                            const float* __restrict__ grad_pol, BwdRow& R, bool& policy) {
  const float t = temperature[row];
  const int64_t tg = target[row];
  const float gr = grad_ref ? grad_ref[row] : 0.0f;
  const float gp = grad_pol ? grad_pol[row] : 0.0f;
  if (gr == 0.0f && gp == 0.0f) return 1;
  const float ref = grad_ref ? ref_logp[row] : 0.0f;
  const int status = grad_pol ? support[row].status : 1;
  const bool invalid = !temperature_valid(t) || tg < 0 || tg >= vocab_real || (ref != ref) || status == -2;
  if (invalid) return 2;
  if (t == 0.0f) return 1;
  if (gp != 0.0f && status == -1) return 2;
  R.c = kLog2e / t;
  R.a_r = grad_ref ? static_cast<float>(-static_cast<double>(lse[row]) * 1.4426950408889634) : 0.0f;
  R.s_r = -gr / t;
  const float gpe = (status == 1) ? gp : 0.0f;
  R.s_p = -gpe / t;
  R.a_p = 0.0f;
  R.thr = INFINITY;
  float tpol = 0.0f;
  if (gpe != 0.0f) {
    const rlk_support_state st = support[row];
    R.a_p = static_cast<float>(-static_cast<double>(st.lse_support) * 1.4426950408889634);
    R.thr = st.threshold;
    tpol = gpe * -expm1f(policy_logp[row]);
  }
  const float tref = (gr != 0.0f) ? gr * -expm1f(ref) : 0.0f;
  R.g_t = (tref + tpol) / t;
  R.vt = tg / 8;
  R.et = static_cast<int>(tg % 8);
  policy = gpe != 0.0f;
  return 0;
}

__global__ __launch_bounds__(kBwdThreads) void k_backward(
    const uint16_t* __restrict__ logits, int64_t row_stride, int64_t vocab_real, int64_t vocab_padded,
    const float* __restrict__ temperature, const int64_t* __restrict__ target, const float* __restrict__ ref_logp,
    const float* __restrict__ lse, const float* __restrict__ grad_ref, const float* __restrict__ policy_logp,
    const rlk_support_state* __restrict__ support, const float* __restrict__ grad_pol,
    uint16_t* __restrict__ grad_out, int64_t grad_stride, int64_t chunks, int64_t n_items) {
  const int64_t nv = vocab_padded / 8;
  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {  // uniform across the workgroup
    const int64_t row = item / chunks;
    const int64_t v0 = (item % chunks) * kBwdChunk;
    const int64_t v1 = (v0 + kBwdChunk < nv) ? v0 + kBwdChunk : nv;
    uint16_t* __restrict__ outp = grad_out + row * grad_stride;
    BwdRow R;
    bool policy = false;
    const int mode = backward_row(row, vocab_real, temperature, target, ref_logp, lse, grad_ref, policy_logp,
                                  support, grad_pol, R, policy);
    if (mode == 1) {
      fill_chunk(outp, vocab_real, v0, v1, 0u);
    } else if (mode == 2) {
      fill_chunk(outp, vocab_real, v0, v1, 0x7FC07FC0u);
    } else if (policy) {
      grad_chunk<true>(logits + row * row_stride, outp, vocab_real, v0, v1, R);
    } else {
      grad_chunk<false>(logits + row * row_stride, outp, vocab_real, v0, v1, R);
    }
  }
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
constexpr int64_t kMaxVocab = int64_t(1) << 30;
constexpr int64_t kMaxNucleusVocab = (int64_t(1) << 24) - (int64_t(1) << 20);  // vocab_real limit of rlk_logp_nucleus
constexpr int64_t kMaxRows = int64_t(1) << 22;       // one workgroup per row: rows * 1024 threads < 2^32
constexpr int64_t kMaxBwdBlocks = int64_t(1) << 21;  // backward grid cap; larger jobs loop over items

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static int32_t check_layout(int64_t n_rows, const rlk_vocab_layout* L) {
  if (L == nullptr) return RLK_ERR_NULL;
  if (n_rows < 0 || n_rows > kMaxRows) return RLK_ERR_SHAPE;
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

static size_t summary_bytes_all(int64_t n_rows) { return static_cast<size_t>(n_rows) * kShards * sizeof(ShardSummary); }

static size_t workspace_bytes(int64_t n_rows, const rlk_vocab_layout* L, bool /*nucleus*/) {
  if (L->groups == 1) return 0;
  return summary_bytes_all(n_rows);
}

static int32_t launched() { return hipGetLastError() == hipSuccess ? RLK_OK : RLK_ERR_HIP; }

// ----------------------------------------------------------------------------
// Static scratch of rlk_logp_nucleus_noalloc: the shard summaries of up to
// kScratchRows rows (groups > 1), in a device array that every GPU the library
// runs on holds until the process ends. In host code `scratch` is only a
// stand-in for the symbol; its device address on each GPU comes from
// hipGetSymbolAddress, taken once per device with that device current.
// ----------------------------------------------------------------------------
constexpr int64_t kScratchRows = RLK_NOALLOC_MAX_ROWS;
static __device__ __align__(256) ShardSummary scratch[kScratchRows * kShards];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (nullptr on a HIP error).
static ShardSummary* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return static_cast<ShardSummary*>(g_scratch_ptr[dev]);
}

// groups > 1: every rank's summaries of the full rows, rank-major, into ws
// (with top_p / top_k: of the rows without a support search only).
static int32_t launch_all_ranks(const uint16_t* logits, int64_t n_rows, const rlk_vocab_layout* L,
                                const float* temperature, const int64_t* target, const float* top_p,
                                const int32_t* top_k, ShardSummary* ws, hipStream_t stream) {
  const int S = static_cast<int>(L->vocab_padded / kShards);
  const int G = L->groups;
  const int spr = kShards / G;
  k_rank_summaries<<<dim3(static_cast<unsigned>(n_rows * G)), dim3(spr * kWave), 0, stream>>>(
      logits, L->row_stride, static_cast<int64_t>(spr) * S, 0, G, spr, S, L->vocab_real, n_rows, temperature, target,
      top_p, top_k, ws);
  return launched();
}

}  // namespace rlk

extern "C" {

const char* rlk_status_string(int32_t status) {
  switch (status) {
    case RLK_OK: return "ok";
    case RLK_ERR_NULL: return "a required pointer is NULL";
    case RLK_ERR_ALIGN: return "misaligned pointer (logits, slices, summaries and workspace need 16 bytes)";
    case RLK_ERR_SHAPE: return "n_rows, rank or a layout field is out of range";
    case RLK_ERR_GROUPS: return "groups must be 1, 2, 4 or 8";
    case RLK_ERR_WORKSPACE: return "workspace or summary buffer missing or too small";
    case RLK_ERR_HIP: return "HIP runtime error while launching";
    case RLK_ERR_SCRATCH: return "n_rows exceeds the static scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

size_t rlk_logp_workspace_bytes(int64_t n_rows, const rlk_vocab_layout* layout, int32_t nucleus) {
  if (rlk::check_layout(n_rows, layout) != RLK_OK) return 0;
  return rlk::workspace_bytes(n_rows, layout, nucleus != 0);
}

size_t rlk_logp_summary_bytes(int64_t n_rows, const rlk_vocab_layout* layout) {
  if (rlk::check_layout(n_rows, layout) != RLK_OK) return 0;
  return rlk::summary_bytes_all(n_rows) / static_cast<size_t>(layout->groups);
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
  if ((st = launch_all_ranks(logits, n_rows, layout, temperature, target, nullptr, nullptr, ws, stream)) != RLK_OK)
    return st;
  const unsigned blocks = static_cast<unsigned>((n_rows + 255) / 256);
  k_merge<<<dim3(blocks), dim3(256), 0, stream>>>(ws, n_rows, kShards / G, S, layout->vocab_real, temperature, target,
                                                  logp_out, lse_out);
  return launched();
}

int32_t rlk_logp_nucleus(const uint16_t* logits, int64_t n_rows, const rlk_vocab_layout* layout,
                         const float* temperature, const float* top_p, const int32_t* top_k, const int64_t* target,
                         float* policy_out, float* ref_out, float* lse_out, rlk_support_state* support_out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace rlk;
  int32_t st = check_layout(n_rows, layout);
  if (st != RLK_OK) return st;
  // support masses are 64-bit integers in units of 2^-40 of 2^R, and a
  // token weighs at most 2^(2^-5) * 2^40 of them (support.hpp,
  // kMaxSupportArg): fewer than 2^24 - 2^20 real tokens keep a row's total
  // below 2^64
  if (layout->vocab_real >= kMaxNucleusVocab) return RLK_ERR_SHAPE;
  if (n_rows == 0) return RLK_OK;  // nothing to read or write: pointers may be NULL
  if (!logits || !temperature || !top_p || !top_k || !target || !policy_out || !ref_out) return RLK_ERR_NULL;
  if (!aligned(logits, 16) || !aligned(temperature, 4) || !aligned(top_p, 4) || !aligned(top_k, 4) ||
      !aligned(target, 8) || !aligned(policy_out, 4) || !aligned(ref_out, 4) || (lse_out && !aligned(lse_out, 4)) ||
      (support_out && !aligned(support_out, 16)))
    return RLK_ERR_ALIGN;
  const size_t need = rlk::workspace_bytes(n_rows, layout, true);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return RLK_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return RLK_ERR_ALIGN;
  }
  const int S = static_cast<int>(layout->vocab_padded / kShards);
  const int G = layout->groups;
  if (G == 1) {
    k_nucleus_g1<false><<<dim3(static_cast<unsigned>(n_rows)), dim3(kNucThreads), 0, stream>>>(
        logits, layout->row_stride, S, layout->vocab_real, temperature, top_p, top_k, target, policy_out, ref_out,
        lse_out, support_out, nullptr, n_rows, kShards);
    return launched();
  }
  ShardSummary* ws = static_cast<ShardSummary*>(workspace);
  if ((st = launch_all_ranks(logits, n_rows, layout, temperature, target, top_p, top_k, ws, stream)) != RLK_OK)
    return st;
  k_nucleus_g1<true><<<dim3(static_cast<unsigned>(n_rows)), dim3(kNucThreads), 0, stream>>>(
      logits, layout->row_stride, S, layout->vocab_real, temperature, top_p, top_k, target, policy_out, ref_out,
      lse_out, support_out, ws, n_rows, kShards / G);
  return launched();
}

int32_t rlk_logp_nucleus_noalloc(const uint16_t* logits, int64_t n_rows, const rlk_vocab_layout* layout,
                                 const float* temperature, const float* top_p, const int32_t* top_k,
                                 const int64_t* target, float* policy_out, float* ref_out, float* lse_out,
                                 rlk_support_state* support_out, hipStream_t stream) {
  using namespace rlk;
  int32_t st = check_layout(n_rows, layout);
  if (st != RLK_OK) return st;
  if (layout->vocab_real >= kMaxNucleusVocab) return RLK_ERR_SHAPE;
  if (layout->groups > 1 && n_rows > kScratchRows) return RLK_ERR_SCRATCH;
  if (n_rows == 0) return RLK_OK;
  if (layout->groups == 1)  // no scratch: the one-launch kernel
    return rlk_logp_nucleus(logits, n_rows, layout, temperature, top_p, top_k, target, policy_out, ref_out,
                            lse_out, support_out, nullptr, 0, stream);
  // the argument checks of rlk_logp_nucleus, before the scratch is looked up
  if (!logits || !temperature || !top_p || !top_k || !target || !policy_out || !ref_out) return RLK_ERR_NULL;
  if (!aligned(logits, 16) || !aligned(temperature, 4) || !aligned(top_p, 4) || !aligned(top_k, 4) ||
      !aligned(target, 8) || !aligned(policy_out, 4) || !aligned(ref_out, 4) || (lse_out && !aligned(lse_out, 4)) ||
      (support_out && !aligned(support_out, 16)))
    return RLK_ERR_ALIGN;
  ShardSummary* ws = scratch_on_current_device();
  if (ws == nullptr) return RLK_ERR_HIP;
  return rlk_logp_nucleus(logits, n_rows, layout, temperature, top_p, top_k, target, policy_out, ref_out, lse_out,
                          support_out, ws, static_cast<size_t>(kScratchRows) * kShards * sizeof(ShardSummary),
                          stream);
}

int32_t rlk_logp_shard_summaries(const uint16_t* logits_slice, int64_t n_rows, const rlk_vocab_layout* layout,
                                 int32_t rank, int64_t slice_stride, const float* temperature,
                                 const int64_t* target, void* summaries_out, size_t summaries_bytes,
                                 hipStream_t stream) {
  using namespace rlk;
  int32_t st = check_layout(n_rows, layout);
  if (st != RLK_OK) return st;
  const int G = layout->groups;
  const int spr = kShards / G;
  const int64_t S = layout->vocab_padded / kShards;
  if (rank < 0 || rank >= G) return RLK_ERR_SHAPE;
  if (slice_stride < spr * S || slice_stride % 8 != 0) return RLK_ERR_SHAPE;
  if (n_rows > 0 && slice_stride > INT64_MAX / 2 / n_rows) return RLK_ERR_SHAPE;
  if (n_rows == 0) return RLK_OK;
  if (!logits_slice || !temperature || !target || !summaries_out) return RLK_ERR_NULL;
  if (!aligned(logits_slice, 16) || !aligned(temperature, 4) || !aligned(target, 8) || !aligned(summaries_out, 16))
    return RLK_ERR_ALIGN;
  if (summaries_bytes < summary_bytes_all(n_rows) / static_cast<size_t>(G)) return RLK_ERR_WORKSPACE;
  k_rank_summaries<<<dim3(static_cast<unsigned>(n_rows)), dim3(spr * kWave), 0, stream>>>(
      logits_slice, slice_stride, 0, rank, 1, spr, static_cast<int>(S), layout->vocab_real, n_rows, temperature,
      target, nullptr, nullptr, static_cast<ShardSummary*>(summaries_out));
  return launched();
}

int32_t rlk_logp_merge(const void* summaries, size_t summaries_bytes, int64_t n_rows,
                       const rlk_vocab_layout* layout, const float* temperature, const int64_t* target,
                       float* logp_out, float* lse_out, hipStream_t stream) {
  using namespace rlk;
  int32_t st = check_layout(n_rows, layout);
  if (st != RLK_OK) return st;
  if (n_rows == 0) return RLK_OK;
  if (!summaries || !temperature || !target || !logp_out) return RLK_ERR_NULL;
  if (!aligned(summaries, 16) || !aligned(temperature, 4) || !aligned(target, 8) || !aligned(logp_out, 4) ||
      (lse_out && !aligned(lse_out, 4)))
    return RLK_ERR_ALIGN;
  if (summaries_bytes < summary_bytes_all(n_rows)) return RLK_ERR_WORKSPACE;
  const int S = static_cast<int>(layout->vocab_padded / kShards);
  const unsigned blocks = static_cast<unsigned>((n_rows + 255) / 256);
  k_merge<<<dim3(blocks), dim3(256), 0, stream>>>(static_cast<const ShardSummary*>(summaries), n_rows,
                                                  kShards / layout->groups, S, layout->vocab_real, temperature, target,
                                                  logp_out, lse_out);
  return launched();
}

int32_t rlk_logp_backward(const uint16_t* logits, int64_t n_rows, const rlk_vocab_layout* layout,
                          const float* temperature, const int64_t* target, const float* ref_logp, const float* lse,
                          const float* grad_ref, const float* policy_logp, const rlk_support_state* support,
                          const float* grad_policy, uint16_t* grad_logits, int64_t grad_stride, hipStream_t stream) {
  using namespace rlk;
  int32_t st = check_layout(n_rows, layout);
  if (st != RLK_OK) return st;
  if (grad_stride < layout->vocab_padded || grad_stride % 8 != 0) return RLK_ERR_SHAPE;
  if (n_rows > 0 && grad_stride > INT64_MAX / 2 / n_rows) return RLK_ERR_SHAPE;
  if (n_rows == 0) return RLK_OK;
  if (!logits || !temperature || !target || !grad_logits) return RLK_ERR_NULL;
  if (!grad_ref && !grad_policy) return RLK_ERR_NULL;
  if (grad_ref && (!ref_logp || !lse)) return RLK_ERR_NULL;
  if (grad_policy && (!policy_logp || !support)) return RLK_ERR_NULL;
  if (!aligned(logits, 16) || !aligned(grad_logits, 16) || !aligned(temperature, 4) || !aligned(target, 8) ||
      (grad_ref && (!aligned(grad_ref, 4) || !aligned(ref_logp, 4) || !aligned(lse, 4))) ||
      (grad_policy && (!aligned(grad_policy, 4) || !aligned(policy_logp, 4) || !aligned(support, 16))))
    return RLK_ERR_ALIGN;
  const int64_t chunks = (layout->vocab_padded / 8 + kBwdChunk - 1) / kBwdChunk;
  const int64_t n_items = n_rows * chunks;
  const int64_t grid = n_items < kMaxBwdBlocks ? n_items : kMaxBwdBlocks;
  k_backward<<<dim3(static_cast<unsigned>(grid)), dim3(kBwdThreads), 0, stream>>>(
      logits, layout->row_stride, layout->vocab_real, layout->vocab_padded, temperature, target,
      grad_ref ? ref_logp : nullptr, grad_ref ? lse : nullptr, grad_ref, grad_policy ? policy_logp : nullptr,
      grad_policy ? support : nullptr, grad_policy, grad_logits, grad_stride, chunks, n_items);
  return launched();
}

}  // extern "C"
