// Device-side building blocks of the strict token-logprob kernels (gfx950, wave64).
//
// Canonical partition (RL-Kernel page "Reproduce and profile the Qwen3-8B
// TP4/CP2 experiment", section "How non-default CUDA topology reuses
// TP4/CP2"): columns [0, vocab_padded) split into 8 virtual shards; each
// shard is reduced to a summary by exactly one wavefront, and the 8 summaries
// are merged left to right. Which workgroup runs which shard-wave never
// changes the arithmetic below, so results do not depend on batch size, row
// position or grouping.
//
// Frozen per-shard order (all integer quantities are per shard):
//   * the shard's real columns form ceil(ncols/8) vectors of 8 BF16 values
//     (16 bytes); vectors 0 .. nfull-1 are complete, a partial last vector
//     (ncols % 8 != 0) is processed after them with its missing columns
//     treated as -inf;
//   * lane l of the wave owns vectors l, l+64, l+128, ...; they are consumed
//     in chunks of U = 8 vectors per lane (chunk j = vectors (jU + u)*64 + l);
//   * each lane keeps 8 accumulators, one per position inside a vector, and
//     adds its terms in vector order;
//   * the lane total is ((a0+a1)+(a2+a3))+((a4+a5)+(a6+a7)); the wave total is
//     an xor butterfly over distances 32,16,8,4,2,1 (commutative adds, so all
//     lanes hold the same bits).
//
// Each term is 2^(x*c - r) with c = fl32(log2(e)/T) and r an integer-valued
// reference exponent shared by the wave: r = ceil(fl32(m0*c)), m0 being the
// exact maximum of the first chunk holding a value above -inf. If the final
// wave total is not below 2^100 (overflow, NaN, or a first chunk far below
// the shard maximum), the shard is recomputed in two passes with r taken from
// the exact shard maximum. Both branches are fixed functions of the shard's
// data, so the result is still one fixed function of the shard.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlk {

constexpr int kWave = 64;
constexpr int kShards = 8;
constexpr uint32_t kNegInfPair = 0xFF80FF80u;  // two BF16 -inf
constexpr float kLog2e = 1.44269504088896340736f;
constexpr double kLn2 = 0.693147180559945309417232121458;
constexpr float kRestartBound = 0x1p100f;

// 16-byte vector of 8 BF16 values (native vector type, so that it can be
// loaded with one 128-bit global load and a non-temporal hint).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Summary of one shard of one row (16 bytes; also the record that ranks of a
// vocabulary-parallel layout exchange).
//   value rows:  r = reference exponent (integer-valued), l = sum of 2^(x*c - r),
//                m = maximum of the first chunk holding a value above -inf (the
//                exact shard maximum when the shard was recomputed),
//                aux = BF16 bits of the target's logit when the target column
//                lies in this shard's real columns, else -1.
//   greedy rows: r = 0, l = 0 (NaN if the shard holds NaN or +inf), m = exact
//                maximum, aux = lowest (global) column holding m, -1 if none.
struct alignas(16) ShardSummary {
  float r;
  float l;
  float m;
  int32_t aux;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) v = v + __shfl_xor(v, d, kWave);
  return v;
}

__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) v = min(v, __shfl_xor(v, d, kWave));
  return v;
}

// Integer-valued reference exponent for a maximum m (log2 units); 0 when the
// maximum is -inf (nothing seen yet).
__device__ __forceinline__ float ref_exponent(float m, float c) {
  return (m == -INFINITY) ? 0.0f : ceilf(m * c);
}

__device__ __forceinline__ bool temperature_valid(float t) {
  return (t >= 0.0f) && (t <= 3.4028234663852886e38f);  // false for NaN and +-inf
}

// Unpack a 16-byte vector into 8 float32 values, in column order.
__device__ __forceinline__ void unpack8(const u32x4& v, float* x) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
  x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// Mask columns >= n (0 < n < 8) of a vector to -inf.
__device__ __forceinline__ u32x4 mask_tail(u32x4 v, int n) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e >= n) {
      uint32_t& word = w[e >> 1];
      word = (e & 1) ? ((word & 0x0000FFFFu) | 0xFF800000u) : ((word & 0xFFFF0000u) | 0x0000FF80u);
    }
  }
  u32x4 out;
  out.x = w[0]; out.y = w[1]; out.z = w[2]; out.w = w[3];
  return out;
}

__device__ __forceinline__ u32x4 neg_inf_vec() {
  u32x4 out;
  out.x = kNegInfPair; out.y = kNegInfPair; out.z = kNegInfPair; out.w = kNegInfPair;
  return out;
}

// Vectors per lane (2048 columns of a shard) whose wave maximum fixes the
// streaming reference: the first such group that holds a value above -inf.
constexpr int kRefGroup = 4;

// Wave-level streaming state for one shard.
struct ShardAcc {
  float acc[8];
  float r;         // reference exponent (wave-uniform)
  bool have_ref;   // wave-uniform
  float m0;        // wave maximum of the chunk that fixed r

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int p = 0; p < 8; ++p) acc[p] = 0.0f;
    r = 0.0f;
    have_ref = false;
    m0 = -INFINITY;
  }

  // Consumes UU vectors; hook(v[u], x, nvalid[u]) sees each vector as loaded
  // and its unpacked values right after their terms are accumulated. Without
  // a hook every vector is widened once, up front; a hook with kLateWiden
  // widens each vector next to its use (the first chunk's maximum from an
  // opaque copy), which keeps the widened values out of the registers the
  // hook needs. Both orders compute the same values.
  template <int UU, typename Hook>
  __device__ __forceinline__ void consume(const u32x4 (&v)[UU], float c, Hook& hook, const int (&nvalid)[UU]) {
    if constexpr (Hook::kLateWiden) {
      consume_late<UU, true, false>(v, c, hook, nvalid);
    } else {
      float x[UU][8];
#pragma unroll
      for (int u = 0; u < UU; ++u) unpack8(v[u], x[u]);
#pragma unroll
      for (int g = 0; g < UU; g += kRefGroup) {
        if (!have_ref) {  // wave-uniform branch, taken until a value above -inf appears
          float cm = -INFINITY;
#pragma unroll
          for (int u = g; u < g + kRefGroup && u < UU; ++u)
#pragma unroll
            for (int p = 0; p < 8; ++p) cm = fmaxf(cm, x[u][p]);
          set_ref(wave_max(cm), c);
        }
      }
      const float nr = -r;
#pragma unroll
      for (int u = 0; u < UU; ++u) {
#pragma unroll
        for (int p = 0; p < 8; ++p) acc[p] += __builtin_amdgcn_exp2f(fmaf(x[u][p], c, nr));
        hook(v[u], x[u], nvalid[u]);
      }
    }
  }

  // The late-widening order. kRef: the reference may still be unset, so each
  // group first checks for it; kFull: every vector holds 8 real columns (the
  // hook's full() sees it and nvalid is not read). Once the reference is set
  // the check is a no-op, so both instantiations compute the same values.
  template <int UU, bool kRef, bool kFull, typename Hook>
  __device__ __forceinline__ void consume_late(const u32x4 (&v)[UU], float c, Hook& hook, const int (&nvalid)[UU]) {
    if constexpr (kRef) {
#pragma unroll
      for (int g = 0; g < UU; g += kRefGroup) {
        if (!have_ref) {  // wave-uniform branch, taken until a value above -inf appears
          float cm = -INFINITY;
#pragma unroll
          for (int u = g; u < g + kRefGroup && u < UU; ++u) {
            u32x4 w = v[u];
            asm volatile("" : "+v"(w));
            float y[8];
            unpack8(w, y);
#pragma unroll
            for (int p = 0; p < 8; ++p) cm = fmaxf(cm, y[p]);
          }
          set_ref(wave_max(cm), c);
        }
      }
    }
    const float nr = -r;
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      float x[8];
      unpack8(v[u], x);
#pragma unroll
      for (int p = 0; p < 8; ++p) acc[p] += __builtin_amdgcn_exp2f(fmaf(x[p], c, nr));
      if constexpr (kFull) {
        hook.full(v[u]);
      } else {
        hook(v[u], x, nvalid[u]);
      }
    }
  }

  // Fixes the reference from the wave maximum of a group of kRefGroup vectors
  // per lane (the first group that holds a value above -inf).
  __device__ __forceinline__ void set_ref(float wm, float c) {
    if (wm > -INFINITY) {
      r = ref_exponent(wm, c);
      m0 = wm;
      have_ref = true;
    }
  }

  __device__ __forceinline__ float lane_total() const {
    return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  }
};

// Loads the chunk starting at vector index `first` (lane offset added here).
template <int U>
__device__ __forceinline__ void load_chunk(const u32x4* __restrict__ base, int first, int nfull, int lane,
                                           u32x4 (&v)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int vi = first + u * kWave + lane;
    v[u] = (vi < nfull) ? __builtin_nontemporal_load(base + vi) : neg_inf_vec();
  }
}

// Per-vector observer called by the streaming pass with each vector as
// loaded, its 8 values (float32 widenings of the BF16 columns, in column
// order) and the number of them that are real columns (8, the tail count, or 0).
struct NoHook {
  static constexpr bool kLateWiden = false;
  __device__ __forceinline__ void operator()(const u32x4&, const float (&)[8], int) const {}
  __device__ __forceinline__ void full(const u32x4&) const {}
};

// No observer, with the register-light order of a hook (for kernels whose
// register budget is set by a hooked pass).
struct NoHookLate : NoHook {
  static constexpr bool kLateWiden = true;
};

// One pass over the shard with the state machine above.
template <int U, typename Hook>
__device__ __forceinline__ void pass_chunk(const u32x4* __restrict__ base, int first, int nfull, int lane, float c,
                                           ShardAcc& st, Hook& hook) {
  u32x4 v[U];
  load_chunk<U>(base, first, nfull, lane, v);
  int nvalid[U];
#pragma unroll
  for (int u = 0; u < U; ++u) nvalid[u] = (first + u * kWave + lane < nfull) ? 8 : 0;
  st.template consume<U>(v, c, hook, nvalid);
}

// With a kLateWiden hook the chunks hold kRefGroup vectors per lane (fewer
// loads in flight per wave, for kernels that run more waves per SIMD). Every
// lane consumes its vectors in the same order and the reference comes from
// the same group in both cases, so the sums are identical. Under such a hook
// the chunks whose vectors are all in range load without bounds checks, and
// after the chunk that fixed the reference they skip its check; the vectors
// after the last whole chunk go one per lane at a time once the reference is
// set. The order of the terms in each accumulator is the same as in the
// guarded loop.
template <int U, typename Hook = NoHook>
__device__ __forceinline__ void shard_pass(const u32x4* __restrict__ base, int nfull, int tail, int lane,
                                           float c, ShardAcc& st, Hook& hook) {
  static_assert(U % kRefGroup == 0, "chunks hold whole reference groups");
  constexpr int kU = Hook::kLateWiden ? kRefGroup : U;
  int first = 0;
  if constexpr (!Hook::kLateWiden) {
    // Whole chunks load without bounds checks (no -inf defaults to select);
    // the reference check stays per group, so the order of the terms and the
    // group that fixes the reference are those of the guarded loop.
    constexpr int kStep = U * kWave;
    const int nmain = nfull - nfull % kStep;
    int all8[U];
#pragma unroll
    for (int u = 0; u < U; ++u) all8[u] = 8;
    for (; first < nmain; first += kStep) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(base + first + u * kWave + lane);
      st.template consume<U>(v, c, hook, all8);
    }
    if (st.have_ref) {
      // The rest one per lane at a time, as under a late-widening hook.
      const int one[1] = {8};
      for (; first < nfull; first += kWave) {
        if (first + lane < nfull) {
          const u32x4 v[1] = {__builtin_nontemporal_load(base + first + lane)};
          st.template consume<1>(v, c, hook, one);
        }
      }
    }
  }
  if constexpr (Hook::kLateWiden) {
    constexpr int kStep = kU * kWave;
    const int nmain = nfull - nfull % kStep;
    const int unused[kU] = {};
    for (; first < nmain && !st.have_ref; first += kStep) {  // wave-uniform condition
      u32x4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = __builtin_nontemporal_load(base + first + u * kWave + lane);
      st.template consume_late<kU, true, true>(v, c, hook, unused);
    }
    if (first < nmain) {
      // The next chunk's loads are issued before this chunk is consumed, so a
      // wave keeps loads in flight while it works; the order of the terms is
      // unchanged.
      u32x4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = __builtin_nontemporal_load(base + first + u * kWave + lane);
      for (; first + kStep < nmain; first += kStep) {
        u32x4 nv[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) nv[u] = __builtin_nontemporal_load(base + first + kStep + u * kWave + lane);
        st.template consume_late<kU, false, true>(v, c, hook, unused);
#pragma unroll
        for (int u = 0; u < kU; ++u) v[u] = nv[u];
      }
      st.template consume_late<kU, false, true>(v, c, hook, unused);
      first += kStep;
    }
    if (st.have_ref) {
      // The rest of the vectors, one per lane at a time. With the reference
      // set, the chunk grouping no longer matters: every accumulator still
      // takes its lane's vectors in order, and the guarded chunk would only
      // have added exact zeros for the missing ones.
      const int one[1] = {0};
      for (; first < nfull; first += kWave) {
        if (first + lane < nfull) {
          const u32x4 v[1] = {__builtin_nontemporal_load(base + first + lane)};
          st.template consume_late<1, false, true>(v, c, hook, one);
        }
      }
    }
  }
  for (; first < nfull; first += kU * kWave) pass_chunk<kU>(base, first, nfull, lane, c, st, hook);
  if (tail) {
    const bool owner = (lane == (nfull & (kWave - 1)));
    u32x4 v[1];
    v[0] = owner ? mask_tail(base[nfull], tail) : neg_inf_vec();
    const int nvalid[1] = {owner ? tail : 0};
    st.template consume<1>(v, c, hook, nvalid);
  }
}

// Exact maximum of the shard (wave-uniform result).
template <int U>
__device__ __forceinline__ float shard_exact_max(const u32x4* __restrict__ base, int nfull, int tail, int lane) {
  float m = -INFINITY;
  for (int first = 0; first < nfull; first += U * kWave) {
    u32x4 v[U];
    load_chunk<U>(base, first, nfull, lane, v);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[8];
      unpack8(v[u], x);
#pragma unroll
      for (int p = 0; p < 8; ++p) m = fmaxf(m, x[p]);
    }
  }
  if (tail && lane == (nfull & (kWave - 1))) {
    float x[8];
    unpack8(mask_tail(base[nfull], tail), x);
#pragma unroll
    for (int p = 0; p < 8; ++p) m = fmaxf(m, x[p]);
  }
  return wave_max(m);
}

// Summary of the shard whose real columns are [col0, col0 + ncols) of `row`,
// for a row with valid temperature T > 0 (c = fl32(log2(e) / T)).
// Must be called by all 64 lanes of a wave.
template <int U, typename Hook = NoHook>
__device__ __forceinline__ ShardSummary summarize_shard(const uint16_t* __restrict__ shard, int ncols, float c,
                                                        Hook& hook) {
  const int lane = threadIdx.x & (kWave - 1);
  const u32x4* __restrict__ base = reinterpret_cast<const u32x4*>(shard);
  const int nfull = ncols >> 3;
  const int tail = ncols & 7;

  ShardAcc st;
  st.init();
  shard_pass<U>(base, nfull, tail, lane, c, st, hook);
  float total = wave_sum(st.lane_total());
  float r = st.r;
  float m = st.m0;

  if (!(total < kRestartBound)) {
    // Two-pass recompute: reference from the exact shard maximum.
    const float mexact = shard_exact_max<U>(base, nfull, tail, lane);
    ShardAcc st2;
    st2.init();
    st2.r = (mexact == INFINITY) ? NAN : ref_exponent(mexact, c);
    st2.have_ref = true;
    NoHook none;
    shard_pass<U>(base, nfull, tail, lane, c, st2, none);
    total = wave_sum(st2.lane_total());
    r = st2.r;
    m = mexact;
    if (!(total < kRestartBound)) total = NAN;  // NaN or +inf logits in the shard
  }
  ShardSummary s;
  s.r = r;
  s.l = total;
  s.m = m;
  s.aux = -1;
  return s;
}

// Greedy (T == 0) summary: exact maximum, its lowest column, and a NaN mark
// when the shard holds NaN or +inf.
// `shard` points at the shard's first column, whose global index is col0.
__device__ __forceinline__ ShardSummary summarize_shard_greedy(const uint16_t* __restrict__ shard, int col0,
                                                              int ncols) {
  const int lane = threadIdx.x & (kWave - 1);
  float m = -INFINITY;
  bool bad = false;
  for (int j = lane; j < ncols; j += kWave) {
    const float x = __uint_as_float(static_cast<uint32_t>(shard[j]) << 16);
    bad |= (x != x) || (x == INFINITY);
    m = fmaxf(m, x);
  }
  m = wave_max(m);
  int first = INT32_MAX;
  for (int j = lane; j < ncols; j += kWave) {
    const float x = __uint_as_float(static_cast<uint32_t>(shard[j]) << 16);
    if (x == m) { first = min(first, col0 + j); break; }
  }
  first = wave_min_i32(first);
  const bool any_bad = __any(bad);
  ShardSummary s;
  s.r = 0.0f;
  s.l = any_bad ? NAN : 0.0f;
  s.m = m;
  s.aux = (first == INT32_MAX) ? -1 : first;
  return s;
}

// Result of merging the 8 shard summaries of one row.
struct RowMerge {
  float logp;     // reference logprob of the target
  float lse;      // natural log-sum-exp of the scaled row (NaN for greedy rows)
  double lse2;    // log2-sum-exp in log2 units (value rows)
  bool ok;        // row produced finite statistics (value rows) / valid greedy result
};

// Fixed-order merge of the 8 summaries of a row (shard 0 first), then the
// target's logprob; the target's logit comes from the aux field of the shard
// holding it (shard_width = columns per shard).
__device__ __forceinline__ RowMerge merge_row(const ShardSummary* __restrict__ s, float t, bool target_ok, int64_t target,
                                              int shard_width) {
  RowMerge out;
  out.logp = NAN;
  out.lse = NAN;
  out.lse2 = NAN;
  out.ok = false;
  if (!temperature_valid(t) || !target_ok) return out;
  if (t == 0.0f) {
    float m = -INFINITY;
    bool bad = false;
#pragma unroll
    for (int k = 0; k < kShards; ++k) {
      m = fmaxf(m, s[k].m);
      bad |= (s[k].l != s[k].l);
    }
    if (bad || m == -INFINITY) return out;
    int first = -1;
#pragma unroll
    for (int k = kShards - 1; k >= 0; --k)  // lowest shard holding the maximum wins
      first = (s[k].m == m) ? s[k].aux : first;
    out.logp = (static_cast<int64_t>(first) == target) ? 0.0f : -INFINITY;
    out.ok = true;
    return out;
  }
  float rmax = -INFINITY;
#pragma unroll
  for (int k = 0; k < kShards; ++k)
    if (s[k].l > 0.0f || s[k].l != s[k].l) rmax = fmaxf(rmax, s[k].r);
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < kShards; ++k) {
    const float l = s[k].l;
    if (l == 0.0f) continue;
    const float d = fmaxf(s[k].r - rmax, -2000.0f);  // <= 0; NaN-free unless r is NaN
    acc = acc + ldexp(static_cast<double>(l), static_cast<int>(d));
    if (s[k].r != s[k].r || l != l) acc = NAN;
  }
  if (!(acc > 0.0) || !(acc < INFINITY) || !(rmax > -INFINITY) || !(rmax < INFINITY)) return out;
  const int ts = static_cast<int>(target / shard_width);
  int tbits = -1;
#pragma unroll
  for (int k = 0; k < kShards; ++k) tbits = (k == ts) ? s[k].aux : tbits;
  if (tbits < 0) return out;  // the shard holding the target did not report it
  const double lse2 = static_cast<double>(rmax) + log2(acc);
  const double lse = lse2 * kLn2;
  const float xt = __uint_as_float(static_cast<uint32_t>(tbits) << 16);
  const float zt = xt / t;  // IEEE float32 division, rounded to nearest
  out.lse2 = lse2;
  out.lse = static_cast<float>(lse);
  out.logp = static_cast<float>(static_cast<double>(zt) - lse);
  out.ok = true;
  return out;
}

}  // namespace rlk
