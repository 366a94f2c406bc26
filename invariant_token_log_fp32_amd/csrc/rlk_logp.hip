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
//   k_nucleus     one workgroup per row: the same merge (reference logprob),
//                 then the top-k/top-p support from integer histograms over a
//                 16-bit monotone key of the BF16 logits, then the policy
//                 logprob.
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

namespace rlk {

// Vectors per lane per chunk in the streaming loop.
constexpr int kChunk = 8;
constexpr int kRowThreads = kShards * kWave;  // 512

// Per-row, per-shard dispatch on the temperature (uniform across the workgroup).
template <bool kExactMax>
__device__ __forceinline__ ShardSummary summarize_row_shard(const uint16_t* __restrict__ rowp, int shard,
                                                            int shard_width, int64_t vocab_real, float t) {
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
  return summarize_shard<kChunk, kExactMax>(rowp, static_cast<int>(col0), ncols, c);
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
  const ShardSummary s = summarize_row_shard<false>(rowp, wave, shard_width, vocab_real, t);
  if ((threadIdx.x & (kWave - 1)) == 0) sm[wave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const RowMerge mr = merge_row(sm, t, tok, tg, xt);
    logp_out[row] = mr.logp;
    if (lse_out) lse_out[row] = mr.lse;
  }
}

template <bool kExactMax>
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
  const ShardSummary s = summarize_row_shard<kExactMax>(rowp, shard, shard_width, vocab_real, t);
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
// Support (top-k, then top-p) from integer histograms.
//
// key16 maps a BF16 bit pattern to a 16-bit integer whose order is the order of
// the float values (and therefore of fl32(x/T) for T > 0), with -0 folded
// into +0. Level-A bins are key >> 4 (4096 bins); a boundary bin is then
// resolved into its 16 keys by a second pass over the row. Counts are exact
// integers; masses are floor(2^(x*c - R) * 2^40) with R = ceil(fl32(M*c)) for
// the exact row maximum M, summed in 64-bit integers. Integer sums do not
// depend on the order of the additions, so the support is the same for any
// schedule of the atomics.
// ----------------------------------------------------------------------------
constexpr int kBinsA = 4096;
constexpr int kSub = 16;

__device__ __forceinline__ uint32_t key16(uint32_t b) {
  b = (b == 0x8000u) ? 0u : b;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

__device__ __forceinline__ unsigned long long fixed40(float w) {
  const uint32_t u = __float_as_uint(w);
  const uint32_t e = u >> 23;  // w >= 0
  const unsigned long long m = static_cast<unsigned long long>((u & 0x7FFFFFu) | 0x800000u);
  const int sh = static_cast<int>(e) - 110;
  if (e == 0 || sh <= -24) return 0ull;
  return sh >= 0 ? (m << sh) : (m >> (-sh));
}

// ceil(p * z) for p in (0, 1) given as a float32, exactly.
__device__ __forceinline__ unsigned long long ceil_mul(float p, unsigned long long z) {
  const uint32_t u = __float_as_uint(p);
  const uint32_t e = u >> 23;
  const uint32_t mant = (e == 0) ? (u & 0x7FFFFFu) : ((u & 0x7FFFFFu) | 0x800000u);
  const int sh = (e == 0) ? 149 : (150 - static_cast<int>(e));  // p = mant * 2^-sh
  const unsigned __int128 a = static_cast<unsigned __int128>(mant) * z;
  if (sh >= 127) return a > 0 ? 1ull : 0ull;
  const unsigned __int128 one = 1;
  return static_cast<unsigned long long>((a + ((one << sh) - 1)) >> sh);
}

struct NucShared {
  uint32_t cnt[kBinsA];
  unsigned long long mass[kBinsA];
  uint32_t sub_cnt[kSub];
  unsigned long long sub_mass[kSub];
  // broadcast state
  int search;
  int k_active;
  int p_active;
  int64_t k;
  float p;
  float c;
  float R;
  int bk;                       // top-k boundary bin (-1 when top-k is off)
  int jk;                       // top-k boundary key inside bk
  uint32_t rc;                  // count of keys >= kappa_k inside bk
  unsigned long long rm;        // mass of keys >= kappa_k inside bk
  int scan_bin;
  uint32_t scan_cnt_above;
  unsigned long long scan_mass_above;
};

// Histogram accumulation for one element (bits of a BF16 logit).
__device__ __forceinline__ void hist_a(NucShared& sh, uint32_t b, float c, float nr) {
  const uint32_t key = key16(b);
  const uint32_t bin = key >> 4;
  atomicAdd(&sh.cnt[bin], 1u);
  const float x = __uint_as_float(b << 16);
  const unsigned long long q = fixed40(__builtin_amdgcn_exp2f(fmaf(x, c, nr)));
  if (q) atomicAdd(&sh.mass[bin], q);
}

__device__ __forceinline__ void hist_b(NucShared& sh, uint32_t b, uint32_t bin_sel, float c, float nr) {
  const uint32_t key = key16(b);
  if ((key >> 4) != bin_sel) return;
  atomicAdd(&sh.sub_cnt[key & 15u], 1u);
  const float x = __uint_as_float(b << 16);
  const unsigned long long q = fixed40(__builtin_amdgcn_exp2f(fmaf(x, c, nr)));
  if (q) atomicAdd(&sh.sub_mass[key & 15u], q);
}

// Whole-row pass applying `f(bits)` to every real column (all threads).
template <typename F>
__device__ __forceinline__ void row_pass(const uint16_t* __restrict__ rowp, int64_t vocab_real, F f) {
  const u32x4* __restrict__ base = reinterpret_cast<const u32x4*>(rowp);
  const int nvec = static_cast<int>(vocab_real >> 3);
  const int tail = static_cast<int>(vocab_real & 7);
  for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
    const u32x4 w = base[v];
    const uint32_t ws4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f(ws4[e] & 0xFFFFu);
      f(ws4[e] >> 16);
    }
  }
  if (tail && threadIdx.x == 0) {
    for (int e = 0; e < tail; ++e) f(static_cast<uint32_t>(rowp[nvec * 8 + e]));
  }
}

template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const T o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

// Wave 0: scan bins from the top (4095 down to 0) and find the first bin where
// the inclusive cumulative count (by_mass = 0) or mass (by_mass = 1) reaches
// `thresh`. Bins above sh.bk count fully, bin sh.bk counts (sh.rc, sh.rm), bins
// below sh.bk count zero (when sh.bk >= 0). Writes scan_bin / *_above.
__device__ void scan_from_top(NucShared& sh, bool by_mass, unsigned long long thresh) {
  const int lane = threadIdx.x & (kWave - 1);
  const int bk = sh.bk;
  auto val = [&](int b, uint32_t& cc, unsigned long long& mm) {
    if (bk < 0 || b > bk) {
      cc = sh.cnt[b];
      mm = sh.mass[b];
    } else if (b == bk) {
      cc = sh.rc;
      mm = sh.rm;
    } else {
      cc = 0;
      mm = 0;
    }
  };
  // lane L covers bins [4095 - 64L - 63, 4095 - 64L]; reads are rotated by lane
  // to spread LDS banks (integer sums, order-free).
  const int hi = kBinsA - 1 - kWave * lane;
  uint32_t tc = 0;
  unsigned long long tm = 0;
  for (int i = 0; i < kWave; ++i) {
    const int b = hi - ((i + lane) & (kWave - 1));
    uint32_t cc;
    unsigned long long mm;
    val(b, cc, mm);
    tc += cc;
    tm += mm;
  }
  const uint32_t ic = wave_incl_scan<uint32_t>(tc, lane);
  const unsigned long long im = wave_incl_scan<unsigned long long>(tm, lane);
  const bool reach = by_mass ? (im >= thresh) : (static_cast<unsigned long long>(ic) >= thresh);
  const unsigned long long ball = __ballot(reach);
  const int L = ball ? __ffsll(static_cast<long long>(ball)) - 1 : kWave - 1;
  const uint32_t ec = __shfl(ic - tc, L, kWave);
  const unsigned long long em = __shfl(im - tm, L, kWave);
  // resolve inside lane L's 64 bins: lane i takes bin (4095 - 64L - i)
  const int b = kBinsA - 1 - kWave * L - lane;
  uint32_t cc;
  unsigned long long mm;
  val(b, cc, mm);
  const uint32_t jc = wave_incl_scan<uint32_t>(cc, lane);
  const unsigned long long jm = wave_incl_scan<unsigned long long>(mm, lane);
  const bool reach2 = by_mass ? (em + jm >= thresh) : (static_cast<unsigned long long>(ec + jc) >= thresh);
  const unsigned long long ball2 = __ballot(reach2);
  const int J = ball2 ? __ffsll(static_cast<long long>(ball2)) - 1 : kWave - 1;
  if (lane == J) {
    sh.scan_bin = b;
    sh.scan_cnt_above = ec + jc - cc;
    sh.scan_mass_above = em + jm - mm;
  }
}

__global__ __launch_bounds__(kRowThreads) void k_nucleus(const uint16_t* __restrict__ logits, int64_t row_stride,
                                                         int64_t vocab_real, const float* __restrict__ temperature,
                                                         const float* __restrict__ top_p,
                                                         const int32_t* __restrict__ top_k,
                                                         const int64_t* __restrict__ target,
                                                         const ShardSummary* __restrict__ ws,
                                                         float* __restrict__ policy_out, float* __restrict__ ref_out) {
  __shared__ NucShared sh;
  const int64_t row = blockIdx.x;
  const uint16_t* __restrict__ rowp = logits + row * row_stride;
  const int tid = threadIdx.x;

  // per-row decisions (thread 0); other threads wait at the barrier
  int64_t tg = -1;
  float ref = NAN, zt = NAN;
  uint32_t key_t = 0;
  double lse2 = NAN;
  if (tid == 0) {
    ShardSummary s[kShards];
#pragma unroll
    for (int k = 0; k < kShards; ++k) s[k] = ws[row * kShards + k];
    const float t = temperature[row];
    tg = target[row];
    const bool tok = (tg >= 0) && (tg < vocab_real);
    uint32_t bt = 0;
    if (tok) bt = rowp[tg];
    const float xt = __uint_as_float(bt << 16);
    const RowMerge mr = merge_row(s, t, tok, tg, xt);
    ref = mr.logp;
    lse2 = mr.lse2;
    ref_out[row] = ref;
    const float p = top_p[row];
    const int64_t k = top_k[row];
    const bool p_ok = (p > 0.0f) && (p <= 1.0f);
    const bool k_ok = (k == -1) || (k >= 1 && k <= vocab_real);
    sh.search = 0;
    float pol;
    if (!mr.ok) {
      pol = NAN;
    } else if (!p_ok || !k_ok) {
      pol = NAN;
    } else if (t == 0.0f) {
      pol = ref;
    } else {
      const bool ka = (k != -1) && (k < vocab_real);
      const bool pa = (p < 1.0f);
      pol = ref;
      if (ka || pa) {
        float m = -INFINITY;
#pragma unroll
        for (int q = 0; q < kShards; ++q) m = fmaxf(m, s[q].m);
        const float c = kLog2e / t;
        sh.search = 1;
        sh.k_active = ka;
        sh.p_active = pa;
        sh.k = k;
        sh.p = p;
        sh.c = c;
        sh.R = ref_exponent(m, c);
        sh.bk = -1;
        sh.rc = 0;
        sh.rm = 0;
        key_t = key16(bt);
        zt = xt / t;
      }
    }
    if (!sh.search) policy_out[row] = pol;
  }
  __syncthreads();
  if (!sh.search) return;

  const float c = sh.c;
  const float nr = -sh.R;
  for (int i = tid; i < kBinsA; i += blockDim.x) {
    sh.cnt[i] = 0;
    sh.mass[i] = 0;
  }
  if (tid < kSub) {
    sh.sub_cnt[tid] = 0;
    sh.sub_mass[tid] = 0;
  }
  __syncthreads();
  row_pass(rowp, vocab_real, [&](uint32_t b) { hist_a(sh, b, c, nr); });
  __syncthreads();

  // top-k: boundary bin by count, then its 16 keys
  int kappa = 0;  // smallest kept key
  uint32_t cnt_s = 0;
  unsigned long long z_k = 0;
  if (sh.k_active) {
    if (tid < kWave) scan_from_top(sh, false, static_cast<unsigned long long>(sh.k));
    __syncthreads();
    const int bk = sh.scan_bin;
    const uint32_t ca = sh.scan_cnt_above;
    const unsigned long long ma = sh.scan_mass_above;
    row_pass(rowp, vocab_real, [&](uint32_t b) { hist_b(sh, b, static_cast<uint32_t>(bk), c, nr); });
    __syncthreads();
    if (tid == 0) {
      uint32_t run = ca;
      unsigned long long rm = 0;
      int j = kSub - 1;
      for (; j >= 0; --j) {
        run += sh.sub_cnt[j];
        rm += sh.sub_mass[j];
        if (static_cast<int64_t>(run) >= sh.k) break;
      }
      j = j < 0 ? 0 : j;
      sh.bk = bk;
      sh.jk = j;
      sh.rc = run - ca;
      sh.rm = rm;
      sh.scan_cnt_above = ca;
      sh.scan_mass_above = ma;
    }
    __syncthreads();
    kappa = sh.bk * kSub + sh.jk;
    cnt_s = sh.scan_cnt_above + sh.rc;
    z_k = sh.scan_mass_above + sh.rm;
  } else {
    // total mass and count of the row
    if (tid < kWave) scan_from_top(sh, false, 0xFFFFFFFFFFFFFFFFull);
    __syncthreads();
    // scan with an unreachable threshold leaves lane 63's bin 0 as the result;
    // totals = above(bin 0) + bin 0
    cnt_s = sh.scan_cnt_above + sh.cnt[0];
    z_k = sh.scan_mass_above + sh.mass[0];
    kappa = 0;
  }

  unsigned long long z_s = z_k;
  if (sh.p_active) {
    const unsigned long long thresh = ceil_mul(sh.p, z_k);
    __syncthreads();
    if (tid < kWave) scan_from_top(sh, true, thresh);
    __syncthreads();
    const int bp = sh.scan_bin;
    const uint32_t ca = sh.scan_cnt_above;
    const unsigned long long ma = sh.scan_mass_above;
    if (!(sh.k_active && bp == sh.bk)) {
      __syncthreads();
      if (tid < kSub) {
        sh.sub_cnt[tid] = 0;
        sh.sub_mass[tid] = 0;
      }
      __syncthreads();
      row_pass(rowp, vocab_real, [&](uint32_t b) { hist_b(sh, b, static_cast<uint32_t>(bp), c, nr); });
      __syncthreads();
    }
    // walk the 16 keys of bp from the top (restricted to keys >= kappa_k)
    const int jlo = (sh.k_active && bp == sh.bk) ? sh.jk : 0;
    uint32_t run_c = ca;
    unsigned long long run_m = ma;
    int j = kSub - 1;
    for (; j > jlo; --j) {
      run_c += sh.sub_cnt[j];
      run_m += sh.sub_mass[j];
      if (run_m >= thresh) break;
    }
    if (j == jlo) {
      run_c += sh.sub_cnt[j];
      run_m += sh.sub_mass[j];
    }
    kappa = bp * kSub + j;
    cnt_s = run_c;
    z_s = run_m;
  }

  if (tid == 0) {
    float pol;
    if (static_cast<int>(key_t) < kappa) {
      pol = -INFINITY;
    } else if (static_cast<int64_t>(cnt_s) == vocab_real) {
      pol = ref;
    } else {
      const double lse_s = (static_cast<double>(sh.R) + (log2(static_cast<double>(z_s)) - 40.0)) * kLn2;
      pol = static_cast<float>(static_cast<double>(zt) - lse_s);
    }
    (void)lse2;
    policy_out[row] = pol;
  }
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

static size_t workspace_bytes(int64_t n_rows, const rlk_vocab_layout* L, bool nucleus) {
  if (!nucleus && L->groups == 1) return 0;
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
  k_summaries<false><<<dim3(static_cast<unsigned>(n_rows * G)), dim3(kShards / G * kWave), 0, stream>>>(
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
  if (!workspace || workspace_bytes < need) return RLK_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return RLK_ERR_ALIGN;
  const int S = static_cast<int>(layout->vocab_padded / kShards);
  const int G = layout->groups;
  ShardSummary* ws = static_cast<ShardSummary*>(workspace);
  k_summaries<true><<<dim3(static_cast<unsigned>(n_rows * G)), dim3(kShards / G * kWave), 0, stream>>>(
      logits, layout->row_stride, S, layout->vocab_real, temperature, G, ws);
  if ((st = launched()) != RLK_OK) return st;
  k_nucleus<<<dim3(static_cast<unsigned>(n_rows)), dim3(kRowThreads), 0, stream>>>(
      logits, layout->row_stride, layout->vocab_real, temperature, top_p, top_k, target, ws, policy_out, ref_out);
  return launched();
}

}  // extern "C"
