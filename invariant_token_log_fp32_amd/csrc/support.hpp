// Top-k / top-p support and policy logprob for one row (one 512-thread workgroup).
//
// Passages: RL-Kernel page "Configurable H100 consistency runs": sampling
// paragraph (top-p in (0, 1], top-k -1 or 1..real vocabulary, support over the
// real vocabulary), mode/KL paragraph (the policy logprob keeps its actual
// top-p/top-k support), command examples (top-k independent of top-p).
//
// Semantics (value thresholds, ties kept): classes are the distinct BF16
// values of the row (-0 folded into +0), in decreasing order. top-k keeps the
// classes down to the first one whose cumulative count reaches k; top-p then
// keeps, among those, the classes down to the first one whose cumulative mass
// reaches p times their total.
//
// Masses are integers: a token of value x weighs floor(2^(x*c - R) * 2^40) with
// c = fl32(log2(e)/T) and R = ceil(fl32(M*c)) for the exact row maximum M; a
// class weighs its count times that. Integer sums are exact and order-free, so
// the support does not depend on the schedule of any atomic; the test
// "cumulative >= p * Z" is evaluated exactly as cumulative >= ceil(p * Z).
//
// Fast path: every token is counted per compressed 16-bit rank (LDS u32
// atomics) in a fixed window of 12288 ranks that covers every BF16 value from
// -4.24e9 to 65536 with magnitude at least 2^-24 (the rank keeps the order of
// the values; -inf tokens are counted apart, mass 0). With groups == 1 the
// shard-waves count while they stream the row for the reference logprob, so
// the support costs no extra pass; otherwise one pass builds it. The row
// maximum is the top non-empty rank, class masses are count * weight, and
// the thresholds come from prefix sums over the window.
// General path, for rows with a token outside the window (including any
// |x| < 2^-24): an exact-maximum pass, then a 4096-bin histogram of
// (count, mass) over key >> 4, then the 16 keys of each boundary bin, each
// from another pass over the row. Both paths produce the same integers and
// therefore the same output bytes.
#pragma once

#include "logp_device.hpp"
#include "rlk_logp.h"

namespace rlk {

constexpr int kNucThreads = 512;
constexpr int kNucWaves = kNucThreads / kWave;
constexpr int kBinsA = 4096;
constexpr int kSub = 16;
constexpr int kWin = 12288;                        // 48 KB of counts: three rows per CU
constexpr int kWinPerThread = kWin / kNucThreads;  // 24
constexpr uint32_t kWinHi = 0x6081u;               // rank of 65536.0: window slot 0
constexpr uint32_t kTinyExp = 103;                 // biased exponent: |x| < 2^-24
constexpr uint32_t kNegInfBits = 0xFF80u;

typedef unsigned long long u64;

// Monotone 16-bit key of a BF16 pattern (-0 folded into +0).
__device__ __forceinline__ uint32_t key16(uint32_t b) {
  b = (b == 0x8000u) ? 0u : b;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

// Compressed rank of a BF16 pattern with |x| >= 2^-24, finite: negative values
// rank 0xFFFF - b (at most 0x4C7F), positive values b + 0x1901 (at least
// 0x4C81); the order of the ranks is the order of the values.
__device__ __forceinline__ uint32_t crank16(uint32_t b) { return (b & 0x8000u) ? (0xFFFFu - b) : (b + 0x1901u); }

// Inverse of crank16.
__device__ __forceinline__ uint32_t crank_bits(uint32_t r) { return (r < 0x4C80u) ? (0xFFFFu - r) : (r - 0x1901u); }

// BF16 value of window slot j (j < kWin).
__device__ __forceinline__ float slot_value(int j) {
  return __uint_as_float(crank_bits(kWinHi - static_cast<uint32_t>(j)) << 16);
}

// BF16 value of a key16 (the +0 key for the folded zeros).
__device__ __forceinline__ float key_value(uint32_t key) {
  const uint32_t b = (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu);
  return __uint_as_float(b << 16);
}

// Window slot of a BF16 pattern (kWinHi - rank), or kWin (the trash slot) for
// -inf, NaN, +-inf, |x| < 2^-24 and values outside the window.
__device__ __forceinline__ uint32_t window_slot(uint32_t b) {
  const uint32_t ex = b & 0x7F80u;
  const bool normal = (ex - (kTinyExp << 7)) < (0x7F80u - (kTinyExp << 7));
  const uint32_t idx = kWinHi - crank16(b);
  return (normal && idx < static_cast<uint32_t>(kWin)) ? idx : static_cast<uint32_t>(kWin);
}

// floor(w * 2^40) for 0 <= w < 2^24 (NaN excluded). Every step is exact: a =
// w * 2^40 is a power-of-two scaling (0 when w is 0 or below the normal range,
// where the floor is 0 as well), hi = floor(a / 2^32) < 2^32 comes from a
// truncating conversion, and a - hi * 2^32 is a multiple of ulp(a) below
// 2^32, so it fits in 24 bits and its truncation is the low word.
__device__ __forceinline__ u64 fixed40(float w) {
  const float a = (w < 0x1p-126f) ? 0.0f : w * 0x1p40f;
  const float hf = a * 0x1p-32f;
  const uint32_t hi = __float2uint_rz(hf);
  const float lo = fmaf(static_cast<float>(hi), -0x1p32f, a);
  return (static_cast<u64>(hi) << 32) | static_cast<u64>(__float2uint_rz(lo));
}

__device__ __forceinline__ u64 weight(uint32_t b, float c, float nr) {
  return fixed40(__builtin_amdgcn_exp2f(fmaf(__uint_as_float(b << 16), c, nr)));
}

// ceil(p * z) for p in (0, 1) given as a float32, exactly.
__device__ __forceinline__ u64 ceil_mul(float p, u64 z) {
  const uint32_t u = __float_as_uint(p);
  const uint32_t e = u >> 23;
  const uint32_t mant = (e == 0) ? (u & 0x7FFFFFu) : ((u & 0x7FFFFFu) | 0x800000u);
  const int sh = (e == 0) ? 149 : (150 - static_cast<int>(e));  // p = mant * 2^-sh
  const unsigned __int128 a = static_cast<unsigned __int128>(mant) * z;
  if (sh >= 127) return a > 0 ? 1ull : 0ull;
  const unsigned __int128 one = 1;
  return static_cast<u64>((a + ((one << sh) - 1)) >> sh);
}

// Integer wave reductions and scans on DPP row operations (VALU only, no LDS
// round trips). Integer sums are exact, so their grouping is free.
// DPP controls: row_shr:n = 0x110 + n, row_ror:n = 0x120 + n, row_bcast:15 =
// 0x142, row_bcast:31 = 0x143.
template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t v) {  // 0 where no source lane / row masked off
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), Ctrl, RowMask, 0xF, true));
}

template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_add(uint32_t v) {
  return v + dpp_or_zero<Ctrl, RowMask>(v);
}

template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ u64 dpp_add(u64 v) {
  const uint32_t lo = dpp_or_zero<Ctrl, RowMask>(static_cast<uint32_t>(v));
  const uint32_t hi = dpp_or_zero<Ctrl, RowMask>(static_cast<uint32_t>(v >> 32));
  return v + ((static_cast<u64>(hi) << 32) | lo);
}

// Inclusive scan over the 64 lanes in lane order: within each row of 16 lanes
// (shifts 1, 2, 4, 8), then row 0's total into row 1 and row 2's running total
// into row 3, then rows 0-1's total into rows 2 and 3.
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v, int /*lane*/) {
  v = dpp_add<0x111>(v);
  v = dpp_add<0x112>(v);
  v = dpp_add<0x114>(v);
  v = dpp_add<0x118>(v);
  v = dpp_add<0x142, 0xA>(v);
  v = dpp_add<0x143, 0xC>(v);
  return v;
}

__device__ __forceinline__ uint32_t lane63(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}
__device__ __forceinline__ u64 lane63(u64 v) {
  return (static_cast<u64>(lane63(static_cast<uint32_t>(v >> 32))) << 32) | lane63(static_cast<uint32_t>(v));
}

// Sum over the wave, in every lane (wave-uniform).
template <typename T>
__device__ __forceinline__ T wave_total(T v) {
  return lane63(wave_incl_scan<T>(v, 0));
}

struct NucGeneral {
  uint32_t cnt[kBinsA];
  u64 mass[kBinsA];
  uint32_t sub_cnt[kSub];
  u64 sub_mass[kSub];
};

struct NucLds {
  ShardSummary sm[kShards];
  // row state, written by thread 0 before the support search
  int search;
  int k_active;
  int p_active;
  int64_t k;
  float p;
  float c;
  float R;
  // block reductions
  uint32_t red_u32[kNucWaves][2];
  u64 red_u64[kNucWaves];
  int red_flag[kNucWaves];
  // search results
  int fast_ok;
  int jk;            // fast: class index of the top-k boundary; general: key inside bk
  uint32_t cnt_k;    // cumulative count through the top-k boundary
  u64 z_k;           // mass of the top-k set
  int kappa;         // support: fast = last kept class index, general = smallest kept key
  int kappa_hi;      // fast: class reached by the upper threshold of a bracketed top-p scan
  uint32_t cnt_s;
  u64 z_s;
  // general path scan state
  int bk;
  uint32_t rc;
  u64 rm;
  int scan_bin;
  uint32_t scan_cnt_above;
  u64 scan_mass_above;
  union {
    uint32_t win[kWin + 1];  // + trash slot
    u64 win_pairs[(kWin + 2) / 2];  // the window (and trash slot) as 64-bit pairs, for clearing
    NucGeneral gen;
  } u;
};

// Applies f(bits) to every real column of the row (all threads of the block).
// Thread t owns vectors t, t + 512, ...; each iteration issues kPassLoads
// independent 128-bit loads before consuming them.
constexpr int kPassLoads = 4;

template <typename F>
__device__ __forceinline__ void row_pass(const uint16_t* __restrict__ rowp, int64_t vocab_real, F f) {
  const u32x4* __restrict__ base = reinterpret_cast<const u32x4*>(rowp);
  const int nvec = static_cast<int>(vocab_real >> 3);
  const int tail = static_cast<int>(vocab_real & 7);
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kNucThreads * kPassLoads) {
    u32x4 w[kPassLoads];
#pragma unroll
    for (int u = 0; u < kPassLoads; ++u) {
      const int vi = v0 + u * kNucThreads;
      w[u] = (vi < nvec) ? base[vi] : neg_inf_vec();
    }
#pragma unroll
    for (int u = 0; u < kPassLoads; ++u) {
      if (v0 + u * kNucThreads < nvec) {
        const uint32_t ws4[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f(ws4[e] & 0xFFFFu);
          f(ws4[e] >> 16);
        }
      }
    }
  }
  if (tail && threadIdx.x == 0) {
    for (int e = 0; e < tail; ++e) f(static_cast<uint32_t>(rowp[nvec * 8 + e]));
  }
}

// As row_pass, but hands whole 16-byte vectors (4 words, 8 values in column
// order) to fv; the partial tail vector's values go one by one to fe.
template <typename FV, typename FE>
__device__ __forceinline__ void row_pass_vec(const uint16_t* __restrict__ rowp, int64_t vocab_real, FV fv, FE fe) {
  const u32x4* __restrict__ base = reinterpret_cast<const u32x4*>(rowp);
  const int nvec = static_cast<int>(vocab_real >> 3);
  const int tail = static_cast<int>(vocab_real & 7);
  const int step = kNucThreads * kPassLoads;
  const int nmain = (nvec / step) * step;
  for (int v0 = threadIdx.x; v0 < nmain; v0 += step) {  // every load in range
    u32x4 w[kPassLoads];
#pragma unroll
    for (int u = 0; u < kPassLoads; ++u) w[u] = base[v0 + u * kNucThreads];
#pragma unroll
    for (int u = 0; u < kPassLoads; ++u) {
      const uint32_t ws4[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
      fv(ws4);
    }
  }
  for (int v = nmain + threadIdx.x; v < nvec; v += kNucThreads) {
    const u32x4 w = base[v];
    const uint32_t ws4[4] = {w.x, w.y, w.z, w.w};
    fv(ws4);
  }
  if (tail && threadIdx.x == 0) {
    for (int e = 0; e < tail; ++e) fe(static_cast<uint32_t>(rowp[nvec * 8 + e]));
  }
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// Window slots of the two BF16 values packed in one 32-bit word, computed on
// 16-bit integer lane pairs (low half = first value):
//   negative b: slot = b - 0x9F7E, in the window iff slot - 0x1402 <= 0x1BFD
//   positive b: slot = 0x4780 - b, in the window iff slot <= 0x1400
// `outside` is nonzero iff a half lies outside the window; halves inside get
// exactly window_slot() (checked against it on all 65536 patterns).
__device__ __forceinline__ uint32_t window_slots2(uint32_t w, uint32_t& outside) {
  uint32_t neg, a, b, slot, lo, d, span;
  asm(
      "v_pk_ashrrev_i16 %[neg], 15, %[w] op_sel_hi:[0,1]\n\t"
      "v_pk_sub_u16 %[a], %[w], %[k1]\n\t"
      "v_pk_sub_u16 %[b], %[k2], %[w]\n\t"
      "v_bfi_b32 %[slot], %[neg], %[a], %[b]\n\t"
      "v_and_b32 %[lo], %[k3], %[neg]\n\t"
      "v_pk_sub_u16 %[d], %[slot], %[lo]\n\t"
      "v_bfi_b32 %[span], %[neg], %[k4], %[k5]\n\t"
      "v_pk_sub_u16 %[out], %[d], %[span] clamp"
      : [neg] "=&v"(neg), [a] "=&v"(a), [b] "=&v"(b), [slot] "=&v"(slot), [lo] "=&v"(lo), [d] "=&v"(d),
        [span] "=&v"(span), [out] "=&v"(outside)
      : [w] "v"(w), [k1] "v"(0x9F7E9F7Eu), [k2] "v"(0x47804780u), [k3] "v"(0x14021402u), [k4] "v"(0x1BFD1BFDu),
        [k5] "v"(0x14001400u));
  return slot;
}

// Window slots of the two BF16 values packed in one 32-bit word, without the
// range check: equal to window_slot() for every half whose value lies in the
// window.
__device__ __forceinline__ uint32_t window_slots2_unchecked(uint32_t w) {
  uint32_t neg, a, b, slot;
  asm(
      "v_pk_ashrrev_i16 %[neg], 15, %[w] op_sel_hi:[0,1]\n\t"
      "v_pk_sub_u16 %[a], %[w], %[k1]\n\t"
      "v_pk_sub_u16 %[b], %[k2], %[w]\n\t"
      "v_bfi_b32 %[slot], %[neg], %[a], %[b]"
      : [neg] "=&v"(neg), [a] "=&v"(a), [b] "=&v"(b), [slot] "=&v"(slot)
      : [w] "v"(w), [k1] "v"(0x9F7E9F7Eu), [k2] "v"(0x47804780u));
  return slot;
}

// Nonzero unless every one of the 8 BF16 values of a vector has magnitude in
// [2^-24, 65536] (patterns 0x3380..0x4780 after the sign is cleared): values
// of either sign in that range lie in the window. A sufficient test only; the
// values it rejects are then slotted one by one.
__device__ __forceinline__ uint32_t vector_outside_core(const uint32_t (&w)[4]) {
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t m = w[i] & 0x7FFF7FFFu;
    asm("v_pk_sub_u16 %0, %1, %2" : "=v"(d[i]) : "v"(m), "v"(0x33803380u));  // wraps below 0x3380
  }
  uint32_t e0, e1, e, out;
  asm(
      "v_pk_max_u16 %[e0], %[d0], %[d1]\n\t"
      "v_pk_max_u16 %[e1], %[d2], %[d3]\n\t"
      "v_pk_max_u16 %[e], %[e0], %[e1]\n\t"
      "v_pk_sub_u16 %[out], %[e], %[span] clamp"
      : [e0] "=&v"(e0), [e1] "=&v"(e1), [e] "=&v"(e), [out] "=&v"(out)
      : [d0] "v"(d[0]), [d1] "v"(d[1]), [d2] "v"(d[2]), [d3] "v"(d[3]), [span] "v"(0x14001400u));
  return out;
}

// Counts tokens into the window while a pass streams them. Per lane: the
// number of -inf tokens and whether any other token fell outside the window.
struct WindowHook {
  static constexpr bool kLateWiden = true;
  uint32_t* win;
  uint32_t ninf;
  bool odd;

  __device__ __forceinline__ explicit WindowHook(uint32_t* w) : win(w), ninf(0), odd(false) {}

  __device__ __forceinline__ void outside(uint32_t b) {
    if (b == kNegInfBits) {
      ++ninf;
    } else {
      odd = true;
    }
  }

  // One by one: the exact slot of each value, or the outside tally.
  __device__ __forceinline__ void each(const uint32_t (&w)[4]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t b = (w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
      const uint32_t slot = window_slot(b);
      if (slot < static_cast<uint32_t>(kWin)) {
        atomicAdd(&win[slot], 1u);
      } else {
        outside(b);
      }
    }
  }

  // A vector of 8 real columns as loaded (column 2i in the low half of word i).
  __device__ __forceinline__ void full(const u32x4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t slots[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) slots[i] = window_slots2_unchecked(w[i]);
    if (vector_outside_core(w) == 0u) {  // all 8 values in the window
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        atomicAdd(&win[slots[i] & 0xFFFFu], 1u);
        atomicAdd(&win[slots[i] >> 16], 1u);
      }
    } else {  // rare: a value that may lie outside the window
      each(w);
    }
  }

  // v: one vector of 8 BF16 columns as loaded (column 2i in the low half of
  // word i); x: their float32 widenings; nvalid of them are real.
  __device__ __forceinline__ void operator()(const u32x4& v, const float (&x)[8], int nvalid) {
    if (nvalid == 8) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t slots[4];
      uint32_t out = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t o;
        slots[i] = window_slots2(w[i], o);
        out |= o;
      }
      if (out == 0u) {  // all 8 values in the window
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          atomicAdd(&win[slots[i] & 0xFFFFu], 1u);
          atomicAdd(&win[slots[i] >> 16], 1u);
        }
      } else {  // rare: a value outside the window, taken one by one
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t b = (w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
          const uint32_t slot = window_slot(b);
          if (slot < static_cast<uint32_t>(kWin)) {
            atomicAdd(&win[slot], 1u);
          } else {
            outside(b);
          }
        }
      }
    } else {
      for (int e = 0; e < nvalid; ++e) {
        const uint32_t b = __float_as_uint(x[e]) >> 16;
        const uint32_t slot = window_slot(b);
        if (slot < static_cast<uint32_t>(kWin)) {
          atomicAdd(&win[slot], 1u);
        } else {
          outside(b);
        }
      }
    }
  }

  // Per-wave totals into L.red_u32[wave][1] (-inf count) and L.red_flag[wave].
  template <typename Lds>
  __device__ __forceinline__ void publish(Lds& L) {
    const uint32_t n = wave_total(ninf);
    const bool any = __any(odd);
    if ((threadIdx.x & (kWave - 1)) == 0) {
      L.red_u32[threadIdx.x / kWave][1] = n;
      L.red_flag[threadIdx.x / kWave] = any;
    }
  }
};

template <typename Lds>
__device__ __forceinline__ void window_clear(Lds& L) {
  for (int i = threadIdx.x; i < (kWin + 2) / 2; i += kNucThreads) L.u.win_pairs[i] = 0ull;
}

// One pass over the row that fills the window (when the streaming pass did not).
__device__ __forceinline__ void window_pass(NucLds& L, const uint16_t* __restrict__ rowp, int64_t vocab_real) {
  WindowHook hook(L.u.win);
  row_pass_vec(rowp, vocab_real,
               [&](const uint32_t (&ws4)[4]) {
                 u32x4 v;
                 v.x = ws4[0]; v.y = ws4[1]; v.z = ws4[2]; v.w = ws4[3];
                 float x[8];
                 unpack8(v, x);
                 hook(v, x, 8);
               },
               [&](uint32_t b) {
                 u32x4 v;
                 v.x = b; v.y = 0u; v.z = 0u; v.w = 0u;
                 const float x[8] = {__uint_as_float(b << 16), 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                 hook(v, x, 1);
               });
  hook.publish(L);
}

template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ int dpp_or_self(int v) {  // own value where no source lane / row masked off
  return __builtin_amdgcn_update_dpp(v, v, Ctrl, RowMask, 0xF, false);
}

// Minimum over the wave, in every lane: rotations inside each row of 16 lanes,
// then the row_bcast steps carry the running minimum to lane 63.
__device__ __forceinline__ int wave_min(int v) {
  v = min(v, dpp_or_self<0x121>(v));
  v = min(v, dpp_or_self<0x122>(v));
  v = min(v, dpp_or_self<0x124>(v));
  v = min(v, dpp_or_self<0x128>(v));
  v = min(v, dpp_or_self<0x142, 0xA>(v));
  v = min(v, dpp_or_self<0x143, 0xC>(v));
  return __builtin_amdgcn_readlane(v, 63);
}

// Block-wide inclusive scan of (count, mass) over the 512 threads, in thread
// order; returns the block totals through tot_c / tot_m. Uses L.red_* (two
// barriers inside).
__device__ __forceinline__ void block_incl_scan(NucLds& L, uint32_t& c, u64& m, uint32_t& tot_c, u64& tot_m) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  c = wave_incl_scan<uint32_t>(c, lane);
  m = wave_incl_scan<u64>(m, lane);
  if (lane == kWave - 1) {
    L.red_u32[wv][0] = c;
    L.red_u64[wv] = m;
  }
  __syncthreads();
  tot_c = 0;
  tot_m = 0;
  for (int w = 0; w < kNucWaves; ++w) {
    const uint32_t wc = L.red_u32[w][0];
    const u64 wm = L.red_u64[w];
    if (w < wv) {
      c += wc;
      m += wm;
    }
    tot_c += wc;
    tot_m += wm;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Fast path on a filled window (L.red_* hold the hook totals). Returns
// (block-uniformly) whether it decided the support; on success L.R is set,
// L.kappa is the last kept class (window slot, or kWin for the -inf class),
// L.cnt_s / L.z_s the support's count and mass, and thread 0's `tclass` the
// target's class.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool support_fast(NucLds& L, int64_t vocab_real, int shard_width, uint32_t bt, int& tclass) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const float c = L.c;

  uint32_t ninf_n = 0;
  bool odd = false;
  for (int w = 0; w < kNucWaves; ++w) {
    ninf_n += L.red_u32[w][1];
    odd |= (L.red_flag[w] != 0);
  }
  if (odd) return false;  // block-uniform

  // the row maximum: first non-empty slot (thread t visits t, t + 512, ...).
  // Every shard summary's m is a token of the row (the maximum of its first
  // chunk, or of the shard), so the row maximum's slot is at most the slot of
  // the largest of them: only the rounds up to that slot are read.
  float mb = -INFINITY;
#pragma unroll
  for (int sh = 0; sh < kShards; ++sh) mb = fmaxf(mb, L.sm[sh].m);
  int r_last = -1;  // block-uniform
  if (mb > -INFINITY)
    r_last = min(static_cast<int>(window_slot(__float_as_uint(mb) >> 16)) / kNucThreads, kWinPerThread - 1);
  int jtop = kWin;
  for (int i = r_last; i >= 0; --i)
    if (L.u.win[i * kNucThreads + tid]) jtop = i * kNucThreads + tid;
  jtop = wave_min(jtop);
  __syncthreads();  // red_* reads above are complete before reuse
  if (lane == 0) L.red_u32[wv][0] = static_cast<uint32_t>(jtop);
  __syncthreads();
  jtop = kWin;
  for (int w = 0; w < kNucWaves; ++w) jtop = min(jtop, static_cast<int>(L.red_u32[w][0]));
  if (jtop == kWin) return false;  // no finite token (cannot happen on a searched row)
  const float m = __uint_as_float(crank_bits(kWinHi - static_cast<uint32_t>(jtop)) << 16);
  const float R = ref_exponent(m, c);
  const float nr = -R;

  // count and mass of class (slot) j; a term below 2^-42 is 0 in 2^-40 fixed point
  auto class_at = [&](int j, uint32_t& cj, u64& mj) {
    cj = L.u.win[j];
    mj = 0;
    if (cj) {
      const float t = fmaf(__uint_as_float(crank_bits(kWinHi - static_cast<uint32_t>(j)) << 16), c, nr);
      if (t >= -42.0f) mj = static_cast<u64>(cj) * fixed40(__builtin_amdgcn_exp2f(t));
    }
  };

  const uint32_t total_c = static_cast<uint32_t>(vocab_real) - ninf_n;

  // Exact total mass of the row (block-uniform result), computed only when a
  // decision needs it. Every real token is in the window or is -inf; masses
  // are summed in 512-slot rounds from the top and stop once a round starts
  // below 2^-42 (slots are in decreasing value order, so every later term is 0).
  auto exact_total = [&]() -> u64 {
    const int r_first = jtop / kNucThreads;
    int r_end = r_first + 1;  // block-uniform: rounds [r_first, r_end) can hold mass
    while (r_end < kWinPerThread &&
           !(fmaf(__uint_as_float(crank_bits(kWinHi - static_cast<uint32_t>(r_end * kNucThreads)) << 16), c, nr) <
             -42.0f))
      ++r_end;
    uint32_t cnt[kWinPerThread];
#pragma unroll
    for (int r = 0; r < kWinPerThread; ++r)
      cnt[r] = (r >= r_first && r < r_end) ? L.u.win[r * kNucThreads + tid] : 0u;
    u64 tm = 0;
#pragma unroll
    for (int r = 0; r < kWinPerThread; ++r) {
      if (cnt[r]) {
        const int j = r * kNucThreads + tid;
        const float t = fmaf(__uint_as_float(crank_bits(kWinHi - static_cast<uint32_t>(j)) << 16), c, nr);
        if (t >= -42.0f) tm += static_cast<u64>(cnt[r]) * fixed40(__builtin_amdgcn_exp2f(t));
      }
    }
    tm = wave_total(tm);
    __syncthreads();
    if (lane == 0) L.red_u64[wv] = tm;
    __syncthreads();
    u64 total_m = 0;
    for (int w = 0; w < kNucWaves; ++w) total_m += L.red_u64[w];
    __syncthreads();
    return total_m;
  };

  // top-k boundary by count (the -inf class when the window holds fewer than k)
  int jk = kWin;
  uint32_t cnt_k = total_c + ninf_n;
  u64 z_k = 0;
  bool z_k_known = false;  // otherwise z_k is the row's total mass, not yet summed
  if (L.k_active) {
    const uint64_t k = static_cast<uint64_t>(L.k);
    if (static_cast<uint64_t>(total_c) >= k) {
      uint32_t carry_c = 0;
      u64 carry_m = 0;
      for (int r = jtop / kNucThreads; r < kWinPerThread; ++r) {  // rounds of 512 slots, from the top
        const int j = r * kNucThreads + tid;
        uint32_t cj;
        u64 mj;
        class_at(j, cj, mj);
        uint32_t ic = cj;
        u64 im = mj;
        uint32_t rc;
        u64 rm;
        block_incl_scan(L, ic, im, rc, rm);
        ic += carry_c;
        im += carry_m;
        const bool hit = static_cast<uint64_t>(ic) >= k && static_cast<uint64_t>(ic - cj) < k;
        if (hit) {
          L.jk = j;
          L.cnt_k = ic;
          L.z_k = im;
        }
        if (static_cast<uint64_t>(carry_c + rc) >= k) break;  // block-uniform
        carry_c += rc;
        carry_m += rm;
      }
      __syncthreads();
      jk = L.jk;
      cnt_k = L.cnt_k;
      z_k = L.z_k;
      z_k_known = true;
      __syncthreads();
    }
  }

  // top-p boundary by mass inside the top-k set: the first class whose
  // cumulative mass reaches P = ceil(p * z_k). Scanning for thresholds
  // p_lo <= P <= p_hi finds classes j_lo <= j* <= j_hi (cumulative masses only
  // grow), so j_lo == j_hi decides j* exactly. Records the hits in L.kappa /
  // L.cnt_s / L.z_s (p_lo) and L.kappa_hi (p_hi); -1 when not reached.
  auto scan_p = [&](u64 p_lo, u64 p_hi) {
    if (tid == 0) {
      L.kappa = -1;
      L.kappa_hi = -1;
    }
    u64 carry_m = 0;
    uint32_t carry_c = 0;
    for (int r = jtop / kNucThreads; r < kWinPerThread; ++r) {
      const int j = r * kNucThreads + tid;
      uint32_t cj;
      u64 mj;
      class_at(j, cj, mj);
      uint32_t ic = cj;
      u64 im = mj;
      uint32_t rc;
      u64 rm;
      block_incl_scan(L, ic, im, rc, rm);  // its barriers order the writes above
      ic += carry_c;
      im += carry_m;
      if (im >= p_lo && (im - mj) < p_lo && j <= jk) {
        L.kappa = j;
        L.cnt_s = ic;
        L.z_s = im;
      }
      if (im >= p_hi && (im - mj) < p_hi && j <= jk) L.kappa_hi = j;
      if (carry_m + rm >= p_hi) break;  // block-uniform
      carry_c += rc;
      carry_m += rm;
    }
    __syncthreads();
  };

  int kappa = jk;
  uint32_t cnt_s = cnt_k;
  u64 z_s = z_k;
  if (L.p_active) {
    bool decided = false;
    if (!z_k_known) {
      // The shard summaries bound the total. Each l_s sums positive float32
      // terms 2^(x*c - r_s) through at most `depth` roundings (a lane's
      // vectors plus a partial one, 3 pairwise levels, 6 butterfly levels):
      // relative error <= depth * 2^-24. A term and the token's integer
      // weight floor(2^(x*c - R) * 2^40) differ by the rounding of their
      // exponent arguments (half an ulp of |x*c - r_s| < 100, since a shard
      // total reaches 2^100 only on the exact-maximum recompute, plus half an
      // ulp of |x*c - R| <= 42 where the weight is nonzero: < 2^-17 relative),
      // by v_exp_f32 (about 2^-23 each), by the floor (under one unit per
      // token on a total of at least 2^39 units) and by terms whose weight
      // floors to 0 (under 1/4 unit each). The bracket takes twice the sum.
      const int depth = (shard_width / 8 + kWave) / kWave + 1 + 3 + 6;
      const double eps = 2.0 * (static_cast<double>(depth) * 0x1p-24 + 0x1p-17 + 0x1p-22 +
                                1.25 * static_cast<double>(vocab_real) * 0x1p-39);
      double zf = 0.0;
#pragma unroll
      for (int sh = 0; sh < kShards; ++sh) {
        const float l = L.sm[sh].l;
        if (l > 0.0f) zf += ldexp(static_cast<double>(l), static_cast<int>(L.sm[sh].r - R) + 40);
      }
      const u64 z_lo = static_cast<u64>(zf * (1.0 - eps));
      const u64 z_hi = static_cast<u64>(zf * (1.0 + eps)) + 1ull;
      scan_p(ceil_mul(L.p, z_lo), ceil_mul(L.p, z_hi));
      decided = (L.kappa >= 0) && (L.kappa == L.kappa_hi);  // block-uniform (LDS, after a barrier)
    }
    if (!decided) {
      if (!z_k_known) {
        z_k = exact_total();
        z_k_known = true;
      }
      const u64 P = ceil_mul(L.p, z_k);
      scan_p(P, P);
    }
    kappa = L.kappa;
    cnt_s = L.cnt_s;
    z_s = L.z_s;
  } else if (!z_k_known) {
    // top-k keeps every finite token and top-p is off: the support is the
    // whole vocabulary, whose policy output is the reference output (the
    // support mass is not used)
    z_s = 0;
  }
  __syncthreads();
  if (tid == 0) {
    L.R = R;
    L.kappa = kappa;
    L.cnt_s = cnt_s;
    L.z_s = z_s;
    tclass = (bt == kNegInfBits) ? kWin : static_cast<int>(window_slot(bt));
  }
  __syncthreads();
  return true;
}

// ---------------------------------------------------------------------------
// General path (any row whose thresholds are not resolved by the fast path).
// ---------------------------------------------------------------------------

// Wave 0: scan level-A bins from the top (4095 down to 0) for the first bin
// where the inclusive cumulative count (by_mass = 0) or mass (by_mass = 1)
// reaches `thresh`. Bins above L.bk count fully, bin L.bk counts (L.rc, L.rm),
// bins below L.bk count zero (when L.bk >= 0).
__device__ __forceinline__ void general_scan(NucLds& L, bool by_mass, u64 thresh) {
  const int lane = threadIdx.x & (kWave - 1);
  const int bk = L.bk;
  auto val = [&](int b, uint32_t& cc, u64& mm) {
    if (bk < 0 || b > bk) {
      cc = L.u.gen.cnt[b];
      mm = L.u.gen.mass[b];
    } else if (b == bk) {
      cc = L.rc;
      mm = L.rm;
    } else {
      cc = 0;
      mm = 0;
    }
  };
  const int hi = kBinsA - 1 - kWave * lane;
  uint32_t tc = 0;
  u64 tm = 0;
  for (int i = 0; i < kWave; ++i) {
    const int b = hi - ((i + lane) & (kWave - 1));  // rotated to spread LDS banks
    uint32_t cc;
    u64 mm;
    val(b, cc, mm);
    tc += cc;
    tm += mm;
  }
  const uint32_t ic = wave_incl_scan<uint32_t>(tc, lane);
  const u64 im = wave_incl_scan<u64>(tm, lane);
  const bool reach = by_mass ? (im >= thresh) : (static_cast<u64>(ic) >= thresh);
  const u64 ball = __ballot(reach);
  const int Ln = ball ? __ffsll(static_cast<long long>(ball)) - 1 : kWave - 1;
  const uint32_t ec = __shfl(ic - tc, Ln, kWave);
  const u64 em = __shfl(im - tm, Ln, kWave);
  const int b = kBinsA - 1 - kWave * Ln - lane;
  uint32_t cc;
  u64 mm;
  val(b, cc, mm);
  const uint32_t jc = wave_incl_scan<uint32_t>(cc, lane);
  const u64 jm = wave_incl_scan<u64>(mm, lane);
  const bool reach2 = by_mass ? (em + jm >= thresh) : (static_cast<u64>(ec + jc) >= thresh);
  const u64 ball2 = __ballot(reach2);
  const int J = ball2 ? __ffsll(static_cast<long long>(ball2)) - 1 : kWave - 1;
  if (lane == J) {
    L.scan_bin = b;
    L.scan_cnt_above = ec + jc - cc;
    L.scan_mass_above = em + jm - mm;
  }
}

__device__ __forceinline__ void general_sub(NucLds& L, const uint16_t* __restrict__ rowp, int64_t vocab_real, uint32_t bin) {
  const float c = L.c;
  const float nr = -L.R;
  if (threadIdx.x < kSub) {
    L.u.gen.sub_cnt[threadIdx.x] = 0;
    L.u.gen.sub_mass[threadIdx.x] = 0;
  }
  __syncthreads();
  row_pass(rowp, vocab_real, [&](uint32_t b) {
    const uint32_t key = key16(b);
    if ((key >> 4) != bin) return;
    atomicAdd(&L.u.gen.sub_cnt[key & 15u], 1u);
    const u64 q = weight(b, c, nr);
    if (q) atomicAdd(&L.u.gen.sub_mass[key & 15u], q);
  });
  __syncthreads();
}

// On return L.R is set, L.kappa is the smallest kept key16, L.cnt_s / L.z_s
// the support's count and mass.
__device__ __forceinline__ void support_general(NucLds& L, const uint16_t* __restrict__ rowp, int64_t vocab_real) {
  const int tid = threadIdx.x;
  const float c = L.c;
  // exact row maximum -> reference exponent R
  float mx = -INFINITY;
  row_pass(rowp, vocab_real, [&](uint32_t b) { mx = fmaxf(mx, __uint_as_float(b << 16)); });
  mx = wave_max(mx);
  if ((tid & (kWave - 1)) == 0) L.red_u32[tid / kWave][0] = __float_as_uint(mx);
  __syncthreads();
  for (int w = 0; w < kNucWaves; ++w) mx = fmaxf(mx, __uint_as_float(L.red_u32[w][0]));
  const float nr = -ref_exponent(mx, c);
  if (tid == 0) L.R = -nr;
  for (int i = tid; i < kBinsA; i += kNucThreads) {
    L.u.gen.cnt[i] = 0;
    L.u.gen.mass[i] = 0;
  }
  if (tid == 0) {
    L.bk = -1;
    L.rc = 0;
    L.rm = 0;
  }
  __syncthreads();
  row_pass(rowp, vocab_real, [&](uint32_t b) {
    const uint32_t bin = key16(b) >> 4;
    atomicAdd(&L.u.gen.cnt[bin], 1u);
    const u64 q = weight(b, c, nr);
    if (q) atomicAdd(&L.u.gen.mass[bin], q);
  });
  __syncthreads();

  int kappa = 0;
  uint32_t cnt_s = 0;
  u64 z_k = 0;
  if (L.k_active) {
    if (tid < kWave) general_scan(L, false, static_cast<u64>(L.k));
    __syncthreads();
    const int bk = L.scan_bin;
    const uint32_t ca = L.scan_cnt_above;
    const u64 ma = L.scan_mass_above;
    general_sub(L, rowp, vocab_real, static_cast<uint32_t>(bk));
    if (tid == 0) {
      uint32_t run = ca;
      u64 rm = 0;
      int j = kSub - 1;
      for (; j >= 0; --j) {
        run += L.u.gen.sub_cnt[j];
        rm += L.u.gen.sub_mass[j];
        if (static_cast<int64_t>(run) >= L.k) break;
      }
      j = j < 0 ? 0 : j;
      L.bk = bk;
      L.jk = j;
      L.rc = run - ca;
      L.rm = rm;
      L.scan_cnt_above = ca;
      L.scan_mass_above = ma;
    }
    __syncthreads();
    kappa = L.bk * kSub + L.jk;
    cnt_s = L.scan_cnt_above + L.rc;
    z_k = L.scan_mass_above + L.rm;
  } else {
    if (tid < kWave) general_scan(L, false, ~0ull);  // unreachable: lands on bin 0
    __syncthreads();
    cnt_s = L.scan_cnt_above + L.u.gen.cnt[0];
    z_k = L.scan_mass_above + L.u.gen.mass[0];
    kappa = 0;
  }
  u64 z_s = z_k;
  if (L.p_active) {
    const u64 thresh = ceil_mul(L.p, z_k);
    __syncthreads();
    if (tid < kWave) general_scan(L, true, thresh);
    __syncthreads();
    const int bp = L.scan_bin;
    const uint32_t ca = L.scan_cnt_above;
    const u64 ma = L.scan_mass_above;
    const bool same = L.k_active && bp == L.bk;
    if (!same) {
      __syncthreads();
      general_sub(L, rowp, vocab_real, static_cast<uint32_t>(bp));
    }
    const int jlo = same ? L.jk : 0;
    uint32_t run_c = ca;
    u64 run_m = ma;
    int j = kSub - 1;
    for (; j > jlo; --j) {
      run_c += L.u.gen.sub_cnt[j];
      run_m += L.u.gen.sub_mass[j];
      if (run_m >= thresh) break;
    }
    if (j == jlo) {
      run_c += L.u.gen.sub_cnt[j];
      run_m += L.u.gen.sub_mass[j];
    }
    kappa = bp * kSub + j;
    cnt_s = run_c;
    z_s = run_m;
  }
  __syncthreads();
  if (tid == 0) {
    L.kappa = kappa;
    L.cnt_s = cnt_s;
    L.z_s = z_s;
  }
  __syncthreads();
}

// Whether a row's policy needs a support search (parameters valid, T > 0, and
// top-k or top-p active); other rows' policy is the reference or NaN.
__device__ __forceinline__ bool search_needed(float t, float p, int64_t k, int64_t vocab_real) {
  const bool p_ok = (p > 0.0f) && (p <= 1.0f);
  const bool k_ok = (k == -1) || (k >= 1 && k <= vocab_real);
  const bool active = (k != -1 && k < vocab_real) || (p < 1.0f);
  return temperature_valid(t) && t != 0.0f && p_ok && k_ok && active;
}

// ---------------------------------------------------------------------------
// Whole-row driver: L.sm must hold the row's 8 shard summaries; when
// `window_built` the window and the hook totals are already filled (the
// streaming pass counted the row). Writes ref_out[row], policy_out[row] and,
// when given, lse_out[row] and state_out[row].
// ---------------------------------------------------------------------------
__device__ __forceinline__ void nucleus_row(NucLds& L, const uint16_t* __restrict__ rowp, int64_t row,
                                            int64_t vocab_real, int shard_width, float t, float p, int64_t k,
                                            int64_t tg, bool window_built, float* __restrict__ policy_out,
                                            float* __restrict__ ref_out, float* __restrict__ lse_out,
                                            rlk_support_state* __restrict__ state_out) {
  const int tid = threadIdx.x;
  float ref = NAN, zt = NAN, lse = NAN;
  uint32_t bt = 0;
  if (tid == 0) {
    const bool tok = (tg >= 0) && (tg < vocab_real);
    const RowMerge mr = merge_row(L.sm, t, tok, tg, shard_width);
    // the target's BF16 bits ride in its shard's summary (a searched row has
    // T > 0 and a successful merge, so that summary reported them)
    if (tok && mr.ok && t > 0.0f) bt = static_cast<uint32_t>(L.sm[tg / shard_width].aux) & 0xFFFFu;
    const float xt = __uint_as_float(bt << 16);
    ref = mr.logp;
    lse = mr.lse;
    ref_out[row] = ref;
    if (lse_out) lse_out[row] = lse;
    const bool p_ok = (p > 0.0f) && (p <= 1.0f);
    const bool k_ok = (k == -1) || (k >= 1 && k <= vocab_real);
    L.search = 0;
    float pol = ref;
    rlk_support_state st;
    st.lse_support = lse;
    st.threshold = -INFINITY;
    st.status = 1;
    st.reserved = 0;
    if (!mr.ok) {
      pol = NAN;
      st.status = -2;
    } else if (!p_ok || !k_ok) {
      pol = NAN;
      st.status = -1;
    } else if (search_needed(t, p, k, vocab_real)) {
      L.search = 1;
      L.k_active = (k != -1) && (k < vocab_real);
      L.p_active = (p < 1.0f);
      L.k = k;
      L.p = p;
      L.c = kLog2e / t;
      zt = xt / t;
    }
    if (!L.search) {
      policy_out[row] = pol;
      if (state_out) state_out[row] = st;
    }
  }
  __syncthreads();
  if (!L.search) return;

  if (!window_built) {
    window_clear(L);
    __syncthreads();
    window_pass(L, rowp, vocab_real);
    __syncthreads();
  }
  int tclass = 0;
  const bool fast = support_fast(L, vocab_real, shard_width, bt, tclass);
  bool in_support;
  if (!fast) {
    __syncthreads();
    support_general(L, rowp, vocab_real);
    in_support = (tid == 0) && static_cast<int>(key16(bt)) >= L.kappa;
  } else {
    in_support = (tid == 0) && tclass <= L.kappa;
  }
  if (tid == 0) {
    const bool whole = static_cast<int64_t>(L.cnt_s) == vocab_real;
    const double lse_s = (static_cast<double>(L.R) + (log2(static_cast<double>(L.z_s)) - 40.0)) * kLn2;
    float pol;
    if (!in_support) {
      pol = -INFINITY;
    } else if (whole) {
      pol = ref;
    } else {
      pol = static_cast<float>(static_cast<double>(zt) - lse_s);
    }
    policy_out[row] = pol;
    if (state_out) {
      rlk_support_state st;
      st.lse_support = whole ? lse : static_cast<float>(lse_s);
      st.threshold = whole ? -INFINITY
                           : (fast ? (L.kappa >= kWin ? -INFINITY : slot_value(L.kappa))
                                   : key_value(static_cast<uint32_t>(L.kappa)));
      st.status = in_support ? 1 : 0;
      st.reserved = 0;
      state_out[row] = st;
    }
  }
}

}  // namespace rlk
