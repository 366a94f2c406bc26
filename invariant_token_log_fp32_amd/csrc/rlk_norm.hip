// Order-independent L2 norm of FP32 gradients (integer exponent bins) for
// gfx950 and the C-ABI declared in include/rlk_norm.h.
//
// Passage: RL-Kernel page "H100 canonical CP backward validation", Change
// section (FP32 gradient squares summed in integer exponent bins before the
// distributed reduction; the norm drives gradient clipping) and Timing and
// scope section (10M-element BF16-derived FP32 norm microbenchmark).
//
// Kernels:
//   k_norm_zero        clears an accumulator (264 words).
//   k_norm_accumulate  streams x with 16-byte non-temporal loads; each lane
//                      pre-sums the squares fl32(x*x) of a 31-binade exponent
//                      window in a 64-bit fixed-point register and adds
//                      everything else (and the register, every 256 terms)
//                      to per-wave LDS copies of the bins with u64 atomics;
//                      at the end the copies are summed and added to the
//                      device bins with u64 atomics. All sums are integer
//                      sums, so the order of the atomics does not matter.
//   k_norm_finalize    one wave: the bins are added exactly into a 384-bit
//                      integer in units of 2^-149 (lane sums, then shuffle
//                      trees over 128-bit group sums and 64-bit limbs),
//                      rounded once to float64 (nearest even); then the
//                      square root. The <true> instance also clears the
//                      accumulator for the next one-call norm.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rlk_logp.h"
#include "rlk_norm.h"

namespace rlk_norm {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 4;                  // 16-byte loads in flight per lane
constexpr int kBins = 256;
constexpr int kWords = sizeof(rlk_norm_bins) / 8;  // 264
constexpr int kMaxBlocks = 256;             // one workgroup per CU
constexpr int64_t kMaxN = int64_t(1) << 39;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64;

struct Counts {
  uint32_t nan;
  uint32_t inf;
};

// Adds the square of one value to the wave's LDS bins directly.
__device__ __forceinline__ void add_square(float v, u64* __restrict__ bins, Counts& c) {
  const float s = v * v;
  const uint32_t u = __float_as_uint(s);
  const uint32_t e = (u >> 23) & 0xFFu;
  const uint32_t frac = u & 0x7FFFFFu;
  if (e == 0xFFu) {
    c.nan += frac != 0u;
    c.inf += frac == 0u;
    return;
  }
  const uint32_t m = frac | (e != 0u ? 0x800000u : 0u);
  if (m != 0u) atomicAdd(&bins[e], static_cast<u64>(m));
}

// Per-lane fixed-point window: squares whose biased exponent e lies in
// [lo, lo + kWin) add m * 2^(e - lo) to one 64-bit register (units of bin lo);
// every other square goes to the LDS bins directly. At most kFlush terms of
// less than 2^(24 + kWin - 1) each are summed before the register is split
// into two 32-bit halves added to bins lo and lo + 32, which keeps the value
// sum_e bin[e] * 2^(max(e,1) - 150) exact while most squares cost no atomic.
constexpr uint32_t kWin = 31;
constexpr int kFlushIters = 16;  // 16 iterations x 16 values = 256 terms < 2^8
constexpr uint32_t kMaxLo = 222;  // lo + 32 <= 254

struct Window {
  uint32_t lo;
  u64 acc;
};

__device__ __forceinline__ void add_square_win(float v, Window& w, u64* __restrict__ bins, Counts& c) {
  const float s = v * v;
  const uint32_t u = __float_as_uint(s);
  const uint32_t e = (u >> 23) & 0xFFu;
  const uint32_t d = e - w.lo;  // wraps for e < lo
  if (d < kWin) {
    w.acc += static_cast<u64>((u & 0x7FFFFFu) | 0x800000u) << d;
  } else {
    add_square(v, bins, c);
  }
}

__device__ __forceinline__ void flush(Window& w, u64* __restrict__ bins) {
  const u64 lo32 = w.acc & 0xFFFFFFFFull;
  const u64 hi32 = w.acc >> 32;
  if (lo32) atomicAdd(&bins[w.lo], lo32);
  if (hi32) atomicAdd(&bins[w.lo + 32], hi32);
  w.acc = 0ull;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t t = __shfl_xor(v, o);
    v = t > v ? t : v;
  }
  return v;
}

__global__ __launch_bounds__(64) void k_norm_zero(u64* __restrict__ bins) {
  for (int i = threadIdx.x; i < kWords; i += 64) bins[i] = 0ull;
}

// 384-bit unsigned integer, little-endian 64-bit limbs. Every limb index
// below is resolved by full unrolling, so the limbs stay in registers.
struct Big {
  u64 w[6];
};

// Limb i of a, 0 outside [0, 6).
__device__ __forceinline__ u64 big_limb(const Big& a, int i) {
  u64 r = 0ull;
#pragma unroll
  for (int k = 0; k < 6; ++k) r = (k == i) ? a.w[k] : r;
  return r;
}

// Bit i of a.
__device__ __forceinline__ u64 big_bit(const Big& a, int i) { return (big_limb(a, i >> 6) >> (i & 63)) & 1ull; }

// Bits [lo, lo + 53) of a as an integer.
__device__ __forceinline__ u64 big_bits53(const Big& a, int lo) {
  const int limb = lo >> 6;
  const int off = lo & 63;
  u64 v = big_limb(a, limb) >> off;
  if (off) v |= big_limb(a, limb + 1) << (64 - off);
  return v & ((1ull << 53) - 1ull);
}

// Any bit below position i set?
__device__ __forceinline__ bool big_any_below(const Big& a, int i) {
  const int limb = i >> 6;
  const int off = i & 63;
  bool any = false;
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const u64 mask = (k < limb) ? ~0ull : (k == limb ? ((off ? (1ull << off) : 1ull) - 1ull) : 0ull);
    any |= (a.w[k] & mask) != 0ull;
  }
  return any;
}

__device__ __forceinline__ u64 readlane64(u64 v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), lane);
  return (static_cast<u64>(hi) << 32) | lo;
}

// Exponent of bin e's unit, in units of 2^-149: the bin counts 24-bit
// significands of squares with biased exponent e, each worth 2^(max(e,1) - 150).
__device__ __forceinline__ int bin_offset(int e) { return e > 0 ? e - 1 : 0; }

// a += v << sh for 128-bit a and v, 0 <= sh < 64 (no overflow by the callers'
// bounds).
__device__ __forceinline__ void add_shl128(u64& a_lo, u64& a_hi, u64 v_lo, u64 v_hi, int sh) {
  const u64 s_lo = v_lo << sh;
  const u64 s_hi = sh ? ((v_hi << sh) | (v_lo >> (64 - sh))) : v_hi;
  const u64 t = a_lo + s_lo;
  a_hi += s_hi + (t < s_lo ? 1ull : 0ull);
  a_lo = t;
}

// The exact sum of the squares from the accumulator words, rounded once to
// float64 (one wave; wave-uniform result). Lane j holds bins 4j .. 4j+3 in
// b[0..3]. Bin e weighs 2^(bin_offset(e)) units of 2^-149.
//   1. Lane j sums its 4 bins at its own offset o_j = bin_offset(4j): shifts
//      of at most 3 bits, so below 2^67 in 128 bits.
//   2. Three shuffle levels add lane j + d into lane j (d = 1, 2, 4, shifted by
//      o_{j+d} - o_j <= 16): lane 8g then holds group g's 32 bins at offset
//      o_{8g}, below 2^98.
//   3. Each group's 128 bits, shifted by o_{8g} mod 64, cover three of the six
//      64-bit limbs of the 384-bit total; per limb, the 8 groups' pieces are
//      added by three more shuffle levels (64-bit sums with carry counts), and
//      lane 0 propagates the carries through the limbs.
// Every step is integer arithmetic, so the total is exact.
__device__ __forceinline__ double exact_sum(const u64 (&b)[4], u64 n_nan, u64 n_inf) {
  if (n_nan != 0ull) return NAN;
  if (n_inf != 0ull) return INFINITY;
  const int lane = threadIdx.x & 63;
  const int o = bin_offset(4 * lane);
  u64 lo = 0ull, hi = 0ull;
#pragma unroll
  for (int i = 0; i < 4; ++i) add_shl128(lo, hi, b[i], 0ull, bin_offset(4 * lane + i) - o);
#pragma unroll
  for (int d = 1; d < 8; d <<= 1) {
    const u64 p_lo = __shfl_down(lo, d);
    const u64 p_hi = __shfl_down(hi, d);
    if ((lane & (2 * d - 1)) == 0) add_shl128(lo, hi, p_lo, p_hi, bin_offset(4 * (lane + d)) - o);
  }
  // lane 8g: group g at offset o (0 for g = 0, 32g - 1 otherwise)
  const int limb0 = o >> 6;
  const int sh = o & 63;
  const u64 q0 = lo << sh;
  const u64 q1 = sh ? ((hi << sh) | (lo >> (64 - sh))) : hi;
  const u64 q2 = sh ? (hi >> (64 - sh)) : 0ull;
  const bool lead = (lane & 7) == 0;
  u64 s_lo[6], s_c[6];
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const u64 piece = (k == limb0) ? q0 : (k == limb0 + 1 ? q1 : (k == limb0 + 2 ? q2 : 0ull));
    s_lo[k] = lead ? piece : 0ull;
    s_c[k] = 0ull;
  }
#pragma unroll
  for (int d = 8; d < 64; d <<= 1) {
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const u64 p_lo = __shfl_down(s_lo[k], d);
      const u64 p_c = __shfl_down(s_c[k], d);
      if ((lane & (2 * d - 1)) == 0) {
        const u64 t = s_lo[k] + p_lo;
        s_c[k] += p_c + (t < p_lo ? 1ull : 0ull);
        s_lo[k] = t;
      }
    }
  }
  Big a;
  u64 carry = 0ull;
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const u64 lk = readlane64(s_lo[k], 0);
    const u64 ck = readlane64(s_c[k], 0);
    const u64 t = lk + carry;
    a.w[k] = t;
    carry = ck + (t < carry ? 1ull : 0ull);
  }
  int top = -1;
#pragma unroll
  for (int i = 0; i < 6; ++i)
    if (a.w[i]) top = 64 * i + 63 - __clzll(static_cast<long long>(a.w[i]));
  if (top < 0) return 0.0;
  if (top < 53) return ldexp(static_cast<double>(a.w[0]), -149);  // exact: fewer than 54 bits
  const int lo_bit = top - 52;
  u64 mant = big_bits53(a, lo_bit);
  const bool round = big_bit(a, lo_bit - 1) != 0ull;
  const bool sticky = big_any_below(a, lo_bit - 1);
  int ex = lo_bit - 149;
  if (round && (sticky || (mant & 1ull))) {
    ++mant;
    if (mant == (1ull << 53)) {
      mant >>= 1;
      ++ex;
    }
  }
  return ldexp(static_cast<double>(mant), ex);
}

// One wave of 64 lanes. Lane l reads words 4l .. 4l+3 (the bins) and lane 0
// the NaN / inf counts; lane 0 writes fl64(S) and fl32(sqrt). With kClear
// every word is then set to 0.
template <bool kClear>
__global__ __launch_bounds__(64) void k_norm_finalize(u64* __restrict__ bins, double* __restrict__ sumsq_out,
                                                      float* __restrict__ norm_out) {
  const int lane = threadIdx.x;
  u64 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = bins[4 * lane + k];
  const u64 n_nan = readlane64(lane == 0 ? bins[kBins] : 0ull, 0);
  const u64 n_inf = readlane64(lane == 0 ? bins[kBins + 1] : 0ull, 0);
  const double s = exact_sum(v, n_nan, n_inf);
  if (lane == 0) {
    if (sumsq_out) *sumsq_out = s;
    if (norm_out) *norm_out = static_cast<float>(sqrt(s));
  }
  if (kClear) {
    for (int i = lane; i < kWords; i += 64) bins[i] = 0ull;
  }
}

// Streams this workgroup's share of x into the per-wave LDS bins (cleared
// here) and the lane's NaN / inf counts. x is 4-byte aligned; elements
// [0, head) precede the first 16-byte boundary, nvec 16-byte vectors follow,
// then `tail` (< 4) elements.
template <int kU>
__device__ __forceinline__ void stream_squares(const float* __restrict__ x, int head, int64_t nvec, int tail,
                                               u64 (&wb)[kWaves][kBins], Counts& c) {
  for (int i = threadIdx.x; i < kWaves * kBins; i += kThreads) (&wb[0][0])[i] = 0ull;
  __syncthreads();
  u64* __restrict__ mine = wb[threadIdx.x / 64];
  if (blockIdx.x == 0) {
    if (static_cast<int>(threadIdx.x) < head) add_square(x[threadIdx.x], mine, c);
    const int tt = static_cast<int>(threadIdx.x) - 64;
    if (tt >= 0 && tt < tail) add_square(x[head + 4 * nvec + tt], mine, c);
  }
  const f32x4* __restrict__ xv = reinterpret_cast<const f32x4*>(x + head);
  const int64_t step = static_cast<int64_t>(gridDim.x) * kThreads * kU;
  Window win = {1u, 0ull};
  int iter = 0;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kU + threadIdx.x; base < nvec;
       base += step) {  // lanes past the end leave at the last step
    f32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * kThreads;
      v[u] = (i < nvec) ? __builtin_nontemporal_load(xv + i) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    if (iter == 0) {
      // window from 28 binades below the largest square the wave's lanes see
      // in their first step; any lo in [1, kMaxLo] is exact, this choice only
      // makes the register path the common one
      uint32_t em = 0u;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float q[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t e = (__float_as_uint(q[k] * q[k]) >> 23) & 0xFFu;
          em = (e != 0xFFu && e > em) ? e : em;
        }
      }
      em = wave_max_u32(em);
      win.lo = em > 29u ? em - 28u : 1u;
      win.lo = win.lo > kMaxLo ? kMaxLo : win.lo;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      add_square_win(v[u].x, win, mine, c);
      add_square_win(v[u].y, win, mine, c);
      add_square_win(v[u].z, win, mine, c);
      add_square_win(v[u].w, win, mine, c);
    }
    iter += kU / 4;
    if (iter >= kFlushIters) {  // at most 16 values per lane per unit of iter since the last flush
      flush(win, mine);
      iter = 1;  // keep the window
    }
  }
  flush(win, mine);
}

// Wave sums of the NaN / inf counts (wave-uniform).
__device__ __forceinline__ void wave_counts(Counts& c) {
  for (int o = 32; o >= 1; o >>= 1) {
    c.nan += __shfl_xor(c.nan, o);
    c.inf += __shfl_xor(c.inf, o);
  }
}

__global__ __launch_bounds__(kThreads) void k_norm_accumulate(const float* __restrict__ x, int head, int64_t nvec,
                                                              int tail, u64* __restrict__ out) {
  __shared__ u64 wb[kWaves][kBins];
  Counts c = {0u, 0u};
  stream_squares<kUnroll>(x, head, nvec, tail, wb, c);
  // NaN / inf counts: wave sums, one atomic per wave when nonzero
  wave_counts(c);
  if ((threadIdx.x & 63) == 0) {
    if (c.nan) atomicAdd(&out[kBins], static_cast<u64>(c.nan));
    if (c.inf) atomicAdd(&out[kBins + 1], static_cast<u64>(c.inf));
  }
  __syncthreads();
  for (int b = threadIdx.x; b < kBins; b += kThreads) {
    u64 s = 0ull;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += wb[w][b];
    if (s) atomicAdd(&out[b], s);
  }
}

static int32_t launched() { return hipGetLastError() == hipSuccess ? RLK_OK : RLK_ERR_HIP; }

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static int32_t launch_accumulate(const float* x, int64_t n, u64* out, hipStream_t stream) {
  int head = n > 0 ? static_cast<int>(((16 - (reinterpret_cast<uintptr_t>(x) & 15)) & 15) / 4) : 0;
  if (head > n) head = static_cast<int>(n);
  const int64_t nvec = (n - head) / 4;
  const int tail = static_cast<int>((n - head) % 4);
  int64_t blocks = (nvec + int64_t(kThreads) * kUnroll - 1) / (int64_t(kThreads) * kUnroll);
  if (blocks < 1) blocks = 1;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  k_norm_accumulate<<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream>>>(x, head, nvec, tail, out);
  return launched();
}

}  // namespace rlk_norm

extern "C" {

int32_t rlk_l2norm_zero(rlk_norm_bins* bins, hipStream_t stream) {
  using namespace rlk_norm;
  if (!bins) return RLK_ERR_NULL;
  if (!aligned(bins, 8)) return RLK_ERR_ALIGN;
  k_norm_zero<<<dim3(1), dim3(64), 0, stream>>>(reinterpret_cast<u64*>(bins));
  return launched();
}

int32_t rlk_l2norm_accumulate(const float* x, int64_t n, rlk_norm_bins* bins, hipStream_t stream) {
  using namespace rlk_norm;
  if (n < 0 || n >= kMaxN) return RLK_ERR_SHAPE;
  if (n == 0) return RLK_OK;
  if (!x || !bins) return RLK_ERR_NULL;
  if (!aligned(x, 4) || !aligned(bins, 8)) return RLK_ERR_ALIGN;
  return launch_accumulate(x, n, reinterpret_cast<u64*>(bins), stream);
}

int32_t rlk_l2norm_finalize(const rlk_norm_bins* bins, double* sumsq_out, float* norm_out, hipStream_t stream) {
  using namespace rlk_norm;
  if (!bins || (!sumsq_out && !norm_out)) return RLK_ERR_NULL;
  if (!aligned(bins, 8) || (sumsq_out && !aligned(sumsq_out, 8)) || (norm_out && !aligned(norm_out, 4)))
    return RLK_ERR_ALIGN;
  k_norm_finalize<false><<<dim3(1), dim3(64), 0, stream>>>(
      reinterpret_cast<u64*>(const_cast<rlk_norm_bins*>(bins)), sumsq_out, norm_out);
  return launched();
}

int32_t rlk_l2norm(const float* x, int64_t n, rlk_norm_bins* workspace, double* sumsq_out, float* norm_out,
                   hipStream_t stream) {
  using namespace rlk_norm;
  if (n < 0 || n >= kMaxN) return RLK_ERR_SHAPE;
  if (!workspace || (!sumsq_out && !norm_out) || (n > 0 && !x)) return RLK_ERR_NULL;
  if ((n > 0 && !aligned(x, 4)) || !aligned(workspace, 8) || (sumsq_out && !aligned(sumsq_out, 8)) ||
      (norm_out && !aligned(norm_out, 4)))
    return RLK_ERR_ALIGN;
  u64* w = reinterpret_cast<u64*>(workspace);
  if (n > 0) {
    const int32_t st = launch_accumulate(x, n, w, stream);
    if (st != RLK_OK) return st;
  }
  k_norm_finalize<true><<<dim3(1), dim3(64), 0, stream>>>(w, sumsq_out, norm_out);
  return launched();
}

}  // extern "C"
