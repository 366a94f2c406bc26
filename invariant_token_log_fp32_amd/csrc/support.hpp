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
// Exact path: every token is counted (LDS u32 atomics) in a window of classes:
// the BF16 values of magnitude in [2^-24, 4096) of either sign, interleaved
// by magnitude (slot 2*(m - m_lo) + sign, m the 15-bit magnitude pattern),
// plus one class for +-0; -inf tokens are counted apart (mass 0). The slots of
// two tokens come from three packed 16-bit instructions, and one maximum over
// a vector's eight slots tells whether all of them lie in the window. Classes
// are visited in value order (positive slots from the largest magnitude down,
// the zero class, negative slots from the smallest magnitude up). The
// shard-waves count while they stream the row, and that is all they do with
// it, whatever the number of physical groups. The row maximum is the largest
// raw pattern the count saw (a signed 16-bit maximum) when the row holds +0 or
// a positive token, else the first non-empty class; class masses are count *
// weight. The eight wavefronts sum the classes' counts and masses in steps
// of 256 classes in parallel; from the step totals one wavefront has the exact
// total Z, finds the steps of the thresholds by prefix sums over the steps,
// and scans only those steps class by class. The same exact total gives the row's reference
// logprob, so a searched row needs no float32 sums at all. A row without a
// search, or whose tokens are not all in the window, or whose maximum is
// beyond the search's range, takes its reference from the float32 shard sums
// instead (a second pass over the row when the first one only counted).
// General path, for rows with a token outside the window (a nonzero value of
// magnitude below 2^-24, or 4096 and beyond): an exact-maximum pass, then a
// 2048-bin histogram of (count, mass) over key >> 5, then the 32 keys of each
// boundary bin, each from another pass over the row. Both paths produce the
// same integers and therefore the same support and policy bytes.
#pragma once

#include "logp_device.hpp"
#include "rlk_logp.h"

namespace rlk {

constexpr int kNucThreads = 512;
constexpr int kNucWaves = kNucThreads / kWave;
constexpr int kBinsA = 2048;  // general path: level-A bins of key16 >> kSubBits
constexpr int kSubBits = 5;
constexpr int kSub = 1 << kSubBits;  // keys per level-A bin
constexpr int kPerLane = kBinsA / kWave;  // level-A bins per lane of the one-wave scan
static_assert(kPerLane * kWave == kBinsA && kPerLane <= kWave && (kPerLane & (kPerLane - 1)) == 0,
              "the scan's lane blocks are whole powers of two");
// The window: magnitudes kMagLo .. kMagLo + kNMag - 1 (2^-24 <= |x| < 4096)
// of both signs, interleaved, then the zero class. 36 KB of counts: four rows
// per CU with the general path's histogram in the same LDS.
constexpr uint32_t kMagLo = 0x3380u;               // magnitude pattern of 2^-24
constexpr int kNMag = 4608;                        // 36 binades of 128 BF16 values
constexpr int kWin = 2 * kNMag;                    // interleaved slots
constexpr int kZeroSlot = kWin;                    // the +-0 class
constexpr int kWinWords = kWin + 2;                // + zero slot + pad (64-bit clearing)
constexpr uint32_t kSlotOut = 0xFFFFFFFFu;         // window_slot() of a token outside the window
// Classes in value order ("ranks"): positives from the top (rank kNMag - 1 - k
// for magnitude index k), the zero class, negatives from the top (rank
// kNMag + 1 + k); kNoRank stands for the -inf class below all of them.
constexpr int kZeroRank = kNMag;
constexpr int kRanks = kWin + 1;
constexpr int kNoRank = kRanks;
constexpr uint32_t kNegInfBits = 0xFF80u;
// Range of the support search: the row maximum's exponent argument
// |fl32(M*c)| < 2^20. Then fl32(M*c) is within 2^-5 of M*c, so no token's
// weight exceeds 2^(2^-5) * 2^40 and, with fewer than 2^24 - 2^20 real tokens
// (the entry points' limit), a row's total mass stays below 2^64. A row beyond
// it gets no support (policy NaN, status -1); its reference comes from the
// float32 shard sums.
constexpr float kMaxSupportArg = 0x1p20f;

typedef unsigned long long u64;

// Monotone 16-bit key of a BF16 pattern (-0 folded into +0).
__device__ __forceinline__ uint32_t key16(uint32_t b) {
  b = (b == 0x8000u) ? 0u : b;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

// BF16 value of a key16 (the +0 key for the folded zeros).
__device__ __forceinline__ float key_value(uint32_t key) {
  const uint32_t b = (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu);
  return __uint_as_float(b << 16);
}

// Window slot of a BF16 pattern: 2 * (m - kMagLo) + sign for magnitudes in the
// window, kZeroSlot for +-0, kSlotOut for everything else (-inf, NaN, +-inf,
// nonzero magnitudes below 2^-24, magnitudes of 4096 and beyond).
__device__ __forceinline__ uint32_t window_slot(uint32_t b) {
  const uint32_t m = b & 0x7FFFu;
  if (m == 0u) return static_cast<uint32_t>(kZeroSlot);
  const uint32_t k = m - kMagLo;  // wraps below kMagLo
  return (k < static_cast<uint32_t>(kNMag)) ? (2u * k + (b >> 15)) : kSlotOut;
}

// Rank (value order) of a window slot.
__device__ __forceinline__ int slot_rank(uint32_t slot) {
  if (slot == static_cast<uint32_t>(kZeroSlot)) return kZeroRank;
  const int k = static_cast<int>(slot >> 1);
  return (slot & 1u) ? (kNMag + 1 + k) : (kNMag - 1 - k);
}

// BF16 pattern and value of the class at a rank (rank < kRanks).
__device__ __forceinline__ uint32_t rank_bits(int r) {
  if (r < kNMag) return kMagLo + static_cast<uint32_t>(kNMag - 1 - r);
  if (r == kZeroRank) return 0u;
  return 0x8000u | (kMagLo + static_cast<uint32_t>(r - kNMag - 1));
}
__device__ __forceinline__ float rank_value(int r) { return __uint_as_float(rank_bits(r) << 16); }

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

// Classes are visited in steps of 256 ranks: the positive slots in 18 steps,
// the zero class alone, the negative slots in 18 steps.
constexpr int kStepRanks = 4 * kWave;           // 256 ranks per step
constexpr int kPosSteps = kNMag / kStepRanks;   // 18
constexpr int kZeroStep = kPosSteps;
constexpr int kSteps = 2 * kPosSteps + 1;
static_assert(kNMag % kStepRanks == 0, "steps cover whole magnitude ranges");
static_assert(kSteps <= kWave, "one lane per step in the step prefix sums");

struct NucLds {
  ShardSummary sm[kShards];
  // row state, written by thread 0 before a block-wide support search
  int search;
  int k_active;
  int p_active;
  int64_t k;
  float p;
  float c;
  float R;
  // block reductions
  uint32_t red_u32[kNucWaves][2];
  int red_flag[kNucWaves];
  int top_w[kNucWaves];  // the row-maximum scan: first non-empty rank per wavefront
  int vmax_w[kNucWaves];  // per wavefront: its largest BF16 pattern read as a signed 16-bit number
  // general path results
  int jk;            // key of the top-k boundary inside bin bk
  int kappa;         // smallest kept key
  uint32_t cnt_s;    // tokens in the support
  u64 z_s;           // support mass
  // general path scan state
  int bk;
  uint32_t rc;
  u64 rm;
  int scan_bin;
  uint32_t scan_cnt_above;
  u64 scan_mass_above;
  int in_range;      // general path: the row maximum lies in the search's range
  // exact path: count and mass of each step of 256 classes, and the target's
  // BF16 pattern
  uint32_t st_c[kSteps];
  u64 st_m[kSteps];
  uint32_t tbits;
  union alignas(16) {
    uint32_t win[kWinWords];        // interleaved slots, the zero class, a pad word
    u64 win_pairs[kWinWords / 2];   // the same as 64-bit pairs, for clearing
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

// Window slots of the two BF16 values packed in one 32-bit word (low half =
// first value), on 16-bit integer lane pairs: the sign bit, then
// 2 * b + sign (the product drops the sign bit, leaving 2 * m + sign), then
// minus 2 * kMagLo. A half lies in the window exactly when its result is below
// kWin: magnitudes below kMagLo wrap to 0x9900 and above, magnitudes of
// kMagLo + kNMag and beyond give kWin .. 0x98FF (no wrap). Halves in the
// window get exactly window_slot() (checked against it on all 65536 patterns).
__device__ __forceinline__ uint32_t window_slots2(uint32_t w) {
  uint32_t sgn, u, slot;
  asm("v_pk_lshrrev_b16 %[sgn], %[c15], %[w]\n\t"
      "v_pk_mad_u16 %[u], %[w], %[c2], %[sgn]\n\t"
      "v_pk_sub_u16 %[slot], %[u], %[lo]"
      : [sgn] "=&v"(sgn), [u] "=&v"(u), [slot] "=&v"(slot)
      : [w] "v"(w), [c15] "v"(0x000F000Fu), [c2] "v"(0x00020002u), [lo] "v"(0x67006700u));
  return slot;
}

// Lane-wise signed 16-bit maximum of two packed pairs. Read as signed 16-bit
// numbers, the BF16 patterns of +0 and the positive values order by value and
// lie above every pattern with the sign bit set, so a running maximum of raw
// patterns that is >= 0 is the pattern of the largest value (checked on the
// host against the value order).
__device__ __forceinline__ uint32_t pk_max_i16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_i16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Nonzero unless all 8 slots of a vector (4 words of slot pairs) are below
// kWin: the packed maximum of the 8, then a saturating subtraction of kWin - 1.
__device__ __forceinline__ uint32_t slots_outside(const uint32_t (&sl)[4]) {
  uint32_t e0, e1, e, out;
  asm("v_pk_max_u16 %[e0], %[s0], %[s1]\n\t"
      "v_pk_max_u16 %[e1], %[s2], %[s3]\n\t"
      "v_pk_max_u16 %[e], %[e0], %[e1]\n\t"
      "v_pk_sub_u16 %[out], %[e], %[top] clamp"
      : [e0] "=&v"(e0), [e1] "=&v"(e1), [e] "=&v"(e), [out] "=&v"(out)
      : [s0] "v"(sl[0]), [s1] "v"(sl[1]), [s2] "v"(sl[2]), [s3] "v"(sl[3]),
        [top] "v"(static_cast<uint32_t>(kWin - 1) * 0x10001u));
  return out;
}

// Counts tokens into the window while a pass streams them. Per lane: the
// number of -inf tokens, whether any other token fell outside the window, and
// the largest raw pattern as a signed 16-bit number (both halves of vmax).
struct WindowHook {
  uint32_t* win;
  uint32_t ninf;
  bool odd;
  uint32_t vmax;

  __device__ __forceinline__ explicit WindowHook(uint32_t* w) : win(w), ninf(0), odd(false), vmax(0x80008000u) {}

  // One token: its exact slot (zero class included), or the outside tally.
  __device__ __forceinline__ void one(uint32_t b) {
    vmax = pk_max_i16(vmax, b * 0x10001u);
    const uint32_t slot = window_slot(b);
    if (slot != kSlotOut) {
      atomicAdd(&win[slot], 1u);
    } else if (b == kNegInfBits) {
      ++ninf;
    } else {
      odd = true;
    }
  }

  // A vector of 8 real columns as loaded (column 2i in the low half of word i).
  __device__ __forceinline__ void full(const u32x4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    vmax = pk_max_i16(vmax, pk_max_i16(pk_max_i16(w[0], w[1]), pk_max_i16(w[2], w[3])));
    uint32_t slots[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) slots[i] = window_slots2(w[i]);
    if (slots_outside(slots) == 0u) {  // all 8 values in the window
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        atomicAdd(&win[slots[i] & 0xFFFFu], 1u);
        atomicAdd(&win[slots[i] >> 16], 1u);
      }
    } else {  // rare: a zero, -inf or a value outside the window, taken one by one
#pragma unroll
      for (int e = 0; e < 8; ++e) one((w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
    }
  }

  // Per-wave totals into L.red_u32[wave][1] (-inf count), L.red_flag[wave]
  // and L.vmax_w[wave].
  template <typename Lds>
  __device__ __forceinline__ void publish(Lds& L) {
    const uint32_t n = wave_total(ninf);
    const bool any = __any(odd);
    const int lo = static_cast<int16_t>(vmax & 0xFFFFu);
    const int hi = static_cast<int16_t>(vmax >> 16);
    int m = lo > hi ? lo : hi;
    for (int d = kWave / 2; d >= 1; d >>= 1) m = max(m, __shfl_xor(m, d, kWave));
    if ((threadIdx.x & (kWave - 1)) == 0) {
      L.red_u32[threadIdx.x / kWave][1] = n;
      L.red_flag[threadIdx.x / kWave] = any;
      L.vmax_w[threadIdx.x / kWave] = m;
    }
  }
};

// One wavefront's pass over its shard of a row that only counts the tokens
// into the window (groups == 1; no float32 sums). Lane l takes the shard's
// 16-byte vectors l, l + 64, ... in chunks of U per lane, and the next chunk's
// loads are issued before the current chunk is counted; the vectors after the
// last whole chunk go in one batch, then the partial vector of the shard's
// last columns. `shard` points at the shard's first column; ncols of its
// columns are real.
template <int U>
__device__ __forceinline__ void count_shard(const uint16_t* __restrict__ shard, int ncols, int lane,
                                            WindowHook& hook) {
  const u32x4* __restrict__ base = reinterpret_cast<const u32x4*>(shard);
  const int nfull = ncols >> 3;
  const int tail = ncols & 7;
  constexpr int kStep = U * kWave;
  const int nmain = nfull - nfull % kStep;
  int first = 0;
  if (nmain > 0) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(base + u * kWave + lane);
    for (; first + kStep < nmain; first += kStep) {
      u32x4 nv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) nv[u] = __builtin_nontemporal_load(base + first + kStep + u * kWave + lane);
#pragma unroll
      for (int u = 0; u < U; ++u) hook.full(v[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = nv[u];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) hook.full(v[u]);
    first = nmain;
  }
  if (first < nfull) {
    const int cnt = (nfull - first + kWave - 1) / kWave;  // at most U vectors per lane, wave-uniform
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int vi = first + u * kWave + lane;
      if (u < cnt && vi < nfull) v[u] = __builtin_nontemporal_load(base + vi);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (u < cnt && first + u * kWave + lane < nfull) hook.full(v[u]);
  }
  if (tail && lane == (nfull & (kWave - 1))) {
    const u32x4 v = base[nfull];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    for (int e = 0; e < tail; ++e) hook.one((w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
  }
}

template <typename Lds>
__device__ __forceinline__ void window_clear(Lds& L) {
  for (int i = threadIdx.x; i < kWinWords / 2; i += kNucThreads) L.u.win_pairs[i] = 0ull;
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

// ---------------------------------------------------------------------------
// Exact path, for a row whose every real token is in the window or is -inf
// (the hook totals say so): all eight wavefronts, then wavefront 0. The row
// maximum M is the first non-empty class, R = ceil(fl32(M*c)), and a class
// weighs count * floor(2^(x*c - R) * 2^40): exactly the integers the general
// path sums per token. The classes are visited in steps of 256 ranks: the
// positive slots in 18 steps, the zero class alone, the negative slots in 18
// steps. In a step lane l holds ranks 4l .. 4l+3 (two 16-byte LDS reads cover
// the 8 interleaved slots of its 4 magnitudes). The wavefronts sum the count
// and the mass of every step from the maximum's on in parallel; one barrier;
// then wavefront 0 has the row's exact total Z from the step totals, and
// prefix sums over the steps locate the step of the top-k boundary (first
// class whose cumulative count reaches k) and of the top-p boundary (first
// class, inside the top-k set, whose cumulative mass reaches ceil(p * Z_k), an
// exact integer test); each of those steps is then scanned class by class (a
// lane-local prefix plus a DPP scan of the lane totals, and a ballot). The
// same total gives the reference logprob: lse = (R + log2(Z) - 40) * ln 2.
// ---------------------------------------------------------------------------

// Rank of element e of lane `lane` in step s (-1 for the unused elements of
// the zero step).
__device__ __forceinline__ int step_rank(int s, int lane, int e) {
  if (s < kPosSteps) return s * kStepRanks + 4 * lane + e;
  if (s == kZeroStep) return (lane == 0 && e == 0) ? kZeroRank : -1;
  return kNMag + 1 + (s - kPosSteps - 1) * kStepRanks + 4 * lane + e;
}

// Step holding a rank (rank < kRanks).
__device__ __forceinline__ int rank_step(int r) {
  if (r < kNMag) return r / kStepRanks;
  if (r == kZeroRank) return kZeroStep;
  return kPosSteps + 1 + (r - kNMag - 1) / kStepRanks;
}

// Counts of the four ranks that `lane` holds in step s.
__device__ __forceinline__ void step_counts(const NucLds& L, int s, int lane, uint32_t (&cnt)[4]) {
  if (s == kZeroStep) {
    cnt[0] = (lane == 0) ? L.u.win[kZeroSlot] : 0u;
    cnt[1] = 0u;
    cnt[2] = 0u;
    cnt[3] = 0u;
  } else if (s < kPosSteps) {
    // ranks r .. r+3 are magnitude indices k .. k-3 (even slots 2k .. 2k-6)
    const int g = 2 * (kNMag - 4) - 8 * (s * kWave + lane);
    const uint4 a = *reinterpret_cast<const uint4*>(&L.u.win[g]);
    const uint4 b = *reinterpret_cast<const uint4*>(&L.u.win[g + 4]);
    cnt[0] = b.z;
    cnt[1] = b.x;
    cnt[2] = a.z;
    cnt[3] = a.x;
  } else {
    // ranks r .. r+3 are negative magnitude indices k .. k+3 (odd slots)
    const int g = 8 * ((s - kPosSteps - 1) * kWave + lane);
    const uint4 a = *reinterpret_cast<const uint4*>(&L.u.win[g]);
    const uint4 b = *reinterpret_cast<const uint4*>(&L.u.win[g + 4]);
    cnt[0] = a.y;
    cnt[1] = a.w;
    cnt[2] = b.y;
    cnt[3] = b.w;
  }
}

__device__ __forceinline__ u64 readlane_u64(u64 v, int l) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), l));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), l));
  return (static_cast<u64>(hi) << 32) | lo;
}

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int l) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
}

// BF16 pattern of the class that `lane` holds as element e of step s (the
// zero step's elements are all the zero class; only lane 0's first one is
// counted there).
__device__ __forceinline__ uint32_t step_bits(int s, int lane, int e) {
  if (s < kPosSteps) return kMagLo + static_cast<uint32_t>(kNMag - 1 - (s * kStepRanks + 4 * lane + e));
  if (s == kZeroStep) return 0u;
  return 0x8000u | (kMagLo + static_cast<uint32_t>((s - kPosSteps - 1) * kStepRanks + 4 * lane + e));
}

// The weight of a class as floor(w * 2^40) = hi * 2^32 + lo (the integers
// fixed40 forms, without its branches): w = 2^(x*c - R) is at most a little
// above 1 for a class at or below the row maximum, so hi <= 256. For an empty
// class above the maximum the parts may be anything; its count is 0.
__device__ __forceinline__ void weight_parts(uint32_t b, float c, float nr, uint32_t& hi, uint32_t& lo) {
  const float w = __builtin_amdgcn_exp2f(fmaf(__uint_as_float(b << 16), c, nr));
  const float a = w * 0x1p40f;  // below 2^-86 for w under the normal range: both parts 0, as in fixed40
  hi = __float2uint_rz(w * 0x1p8f);
  lo = __float2uint_rz(fmaf(static_cast<float>(hi), -0x1p32f, a));
}

// count * floor(w * 2^40) for a count below 2^24 (hi <= 256, so the high part
// is a 24-bit product).
__device__ __forceinline__ u64 class_mass(uint32_t cnt, uint32_t hi, uint32_t lo) {
  const uint32_t hp = static_cast<uint32_t>(__umul24(cnt, hi));  // below 2^32; __umul24 returns int
  return (static_cast<u64>(hp) << 32) + static_cast<u64>(cnt) * lo;
}

// One step, class by class: per-class counts and masses, and the inclusive
// cumulative count and mass of each class counted from the step's first class
// (lane-local prefix plus the exclusive DPP scan of the lanes).
struct StepRound {
  uint32_t cnt[4];
  u64 mass[4];
  uint32_t cum_c[4];
  u64 cum_m[4];
};

__device__ __forceinline__ void step_round(const NucLds& L, int s, float c, float nr, StepRound& Q) {
  const int lane = threadIdx.x & (kWave - 1);
  step_counts(L, s, lane, Q.cnt);
  uint32_t pc = 0;
  u64 pm = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t hi, lo;
    weight_parts(step_bits(s, lane, e), c, nr, hi, lo);
    const u64 m = class_mass(Q.cnt[e], hi, lo);
    Q.mass[e] = m;
    pc += Q.cnt[e];
    pm += m;
    Q.cum_c[e] = pc;
    Q.cum_m[e] = pm;
  }
  const uint32_t ec = wave_incl_scan<uint32_t>(pc, lane) - pc;
  const u64 em = wave_incl_scan<u64>(pm, lane) - pm;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    Q.cum_c[e] += ec;
    Q.cum_m[e] += em;
  }
}

constexpr int kBatch = 4;  // steps per wavefront in the row-maximum scan
static_assert(kBatch * kNucWaves <= kSteps, "the parallel scan covers whole batches of the window");

// First non-empty class among steps s0 .. s0 + kBatch - 1 (steps past the
// window count as empty), kNoRank when they are all empty (wave-uniform). The
// LDS reads of the kBatch steps are issued together; one wave minimum.
__device__ __forceinline__ int batch_top_rank(const NucLds& L, int s0, int lane) {
  uint32_t cn[kBatch][4];
#pragma unroll
  for (int b = 0; b < kBatch; ++b) {
    if (s0 + b < kSteps) {
      step_counts(L, s0 + b, lane, cn[b]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) cn[b][e] = 0u;
    }
  }
  int hit = -1;  // first step of the batch with a token (wave-uniform)
#pragma unroll
  for (int b = kBatch - 1; b >= 0; --b)
    if (__ballot((cn[b][0] | cn[b][1] | cn[b][2] | cn[b][3]) != 0u)) hit = b;
  if (hit < 0) return kNoRank;
  int j = kNoRank;
#pragma unroll
  for (int b = 0; b < kBatch; ++b)
    if (b == hit) {
#pragma unroll
      for (int e = 3; e >= 0; --e)
        if (cn[b][e]) j = step_rank(s0 + b, lane, e);
    }
  return wave_min(j);
}

// Rank of the first non-empty class (the row maximum), kNoRank when the
// window is empty; the same in every thread. Called by the whole block (one
// barrier): wavefront w scans steps kBatch*w .. kBatch*w + kBatch - 1 and the
// minimum over the wavefronts is the answer, so where the maximum lies in the
// window does not lengthen the scan. Only when those steps are all empty (every
// token negative with a magnitude in the last steps) are the remaining steps
// scanned in order.
__device__ __forceinline__ int window_top_rank(NucLds& L, int lane, int wave) {
  const int jw = batch_top_rank(L, kBatch * wave, lane);
  if (lane == 0) L.top_w[wave] = jw;
  __syncthreads();
  int j = kNoRank;
#pragma unroll
  for (int w = 0; w < kNucWaves; ++w) j = min(j, L.top_w[w]);
  for (int s0 = kBatch * kNucWaves; j == kNoRank && s0 < kSteps; s0 += kBatch) j = batch_top_rank(L, s0, lane);
  return j;
}

// Count and mass of one step, summed over the wave (wave-uniform). The
// weights of a step whose classes are all empty, or that lies at or past
// s_end (no class of nonzero weight), are skipped.
__device__ __forceinline__ void step_total(const NucLds& L, int s, int s_end, int lane, float c, float nr,
                                           uint32_t& tc, u64& tm) {
  uint32_t cn[4];
  step_counts(L, s, lane, cn);
  const uint32_t pc = (cn[0] + cn[1]) + (cn[2] + cn[3]);
  uint32_t sum_hi = 0u;  // sum of count * hi: below 2^24 * 256 over a row
  u64 sum_lo = 0ull;
  if (s < s_end && __ballot(pc != 0u)) {  // wave-uniform
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t hi, lo;
      weight_parts(step_bits(s, lane, e), c, nr, hi, lo);
      sum_hi += static_cast<uint32_t>(__umul24(cn[e], hi));
      sum_lo += static_cast<u64>(cn[e]) * lo;
    }
  }
  tc = wave_total<uint32_t>(pc);
  tm = wave_total<u64>((static_cast<u64>(sum_hi) << 32) + sum_lo);
}


// ---------------------------------------------------------------------------
// General path (any row whose thresholds are not resolved by the fast path).
// ---------------------------------------------------------------------------

// Wave 0: scan level-A bins from the top (kBinsA - 1 down to 0) for the first bin
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
  const int hi = kBinsA - 1 - kPerLane * lane;
  uint32_t tc = 0;
  u64 tm = 0;
#pragma unroll 1
  for (int i = 0; i < kPerLane; ++i) {
    const int b = hi - ((i + lane) & (kPerLane - 1));  // rotated to spread LDS banks
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
  // the kPerLane bins of lane Ln's block, one per lane (the other lanes hold none)
  const int b = kBinsA - 1 - kPerLane * Ln - (lane < kPerLane ? lane : kPerLane - 1);
  uint32_t cc = 0;
  u64 mm = 0;
  if (lane < kPerLane) val(b, cc, mm);
  const uint32_t jc = wave_incl_scan<uint32_t>(cc, lane);
  const u64 jm = wave_incl_scan<u64>(mm, lane);
  const bool reach2 = by_mass ? (em + jm >= thresh) : (static_cast<u64>(ec + jc) >= thresh);
  const u64 ball2 = __ballot(reach2 && lane < kPerLane);
  const int J = ball2 ? __ffsll(static_cast<long long>(ball2)) - 1 : kPerLane - 1;
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
    if ((key >> kSubBits) != bin) return;
    atomicAdd(&L.u.gen.sub_cnt[key & (kSub - 1u)], 1u);
    const u64 q = weight(b, c, nr);
    if (q) atomicAdd(&L.u.gen.sub_mass[key & (kSub - 1u)], q);
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
  if (tid == 0) {
    L.R = -nr;
    L.in_range = fabsf(mx * c) < kMaxSupportArg;
  }
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
    const uint32_t bin = key16(b) >> kSubBits;
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
// Row drivers.
// ---------------------------------------------------------------------------

// Merge of the row's summaries and what it decides: the reference logprob,
// the target's BF16 bits, and whether the row needs a support search
// (status 0), takes the reference as its policy (1), or is invalid (-1: top-p
// or top-k out of range; -2: the reference itself failed).
struct RowStart {
  float ref;
  float lse;
  uint32_t bt;
  int status;
};

__device__ __forceinline__ RowStart row_start(const ShardSummary* __restrict__ sm, int64_t vocab_real,
                                              int shard_width, float t, float p, int64_t k, int64_t tg) {
  RowStart rs;
  const bool tok = (tg >= 0) && (tg < vocab_real);
  const RowMerge mr = merge_row(sm, t, tok, tg, shard_width);
  rs.bt = 0;
  // the target's BF16 bits ride in its shard's summary (a searched row has
  // T > 0 and a successful merge, so that summary reported them)
  if (tok && mr.ok && t > 0.0f) rs.bt = static_cast<uint32_t>(sm[tg / shard_width].aux) & 0xFFFFu;
  rs.ref = mr.logp;
  rs.lse = mr.lse;
  const bool p_ok = (p > 0.0f) && (p <= 1.0f);
  const bool k_ok = (k == -1) || (k >= 1 && k <= vocab_real);
  if (!mr.ok) {
    rs.status = -2;
  } else if (!p_ok || !k_ok) {
    rs.status = -1;
  } else {
    rs.status = search_needed(t, p, k, vocab_real) ? 0 : 1;
  }
  return rs;
}

// Outputs of a row that needs no search (status != 0).
__device__ __forceinline__ void write_unsearched(int64_t row, const RowStart& rs, float* __restrict__ policy_out,
                                                 rlk_support_state* __restrict__ state_out) {
  rlk_support_state st;
  st.lse_support = rs.lse;
  st.threshold = -INFINITY;
  st.status = (rs.status == 1) ? 1 : rs.status;
  st.reserved = 0;
  policy_out[row] = (rs.status == 1) ? rs.ref : NAN;
  if (state_out) state_out[row] = st;
}

// Policy logprob and support record of a searched row. `fast`: kappa is a
// rank (kNoRank = the -inf class); otherwise a key16 (general path).
// A row whose maximum lies outside the search's range (!in_range) is written
// as a row without a support: policy NaN, status -1.
__device__ __forceinline__ void write_policy(int64_t row, int64_t vocab_real, bool fast, int kappa, uint32_t cnt_s,
                                             u64 z_s, float R, bool in_range, const RowStart& rs, float t,
                                             float* __restrict__ policy_out, rlk_support_state* __restrict__ state_out) {
  if (!in_range) {
    RowStart none = rs;
    none.status = -1;
    write_unsearched(row, none, policy_out, state_out);
    return;
  }
  const uint32_t bt = rs.bt;
  const int trank = (bt == kNegInfBits) ? kNoRank : slot_rank(window_slot(bt));
  const bool in_support = fast ? (trank <= kappa) : (static_cast<int>(key16(bt)) >= kappa);
  const float zt = __uint_as_float(bt << 16) / t;  // IEEE float32 division
  const bool whole = static_cast<int64_t>(cnt_s) == vocab_real;
  const double lse_s = (static_cast<double>(R) + (log2(static_cast<double>(z_s)) - 40.0)) * kLn2;
  float pol;
  if (!in_support) {
    pol = -INFINITY;
  } else if (whole) {
    pol = rs.ref;
  } else {
    pol = static_cast<float>(static_cast<double>(zt) - lse_s);
  }
  policy_out[row] = pol;
  if (state_out) {
    rlk_support_state st;
    st.lse_support = whole ? rs.lse : static_cast<float>(lse_s);
    st.threshold = whole ? -INFINITY
                         : (fast ? (kappa >= kNoRank ? -INFINITY : rank_value(kappa))
                                 : key_value(static_cast<uint32_t>(kappa)));
    st.status = in_support ? 1 : 0;
    st.reserved = 0;
    state_out[row] = st;
  }
}

// Outputs of a row that needs no search, in wavefront 0 (lane 0 writes): the
// merge of the shard summaries gives the reference, and the policy is the
// reference or NaN.
__device__ __forceinline__ void unsearched_row(const NucLds& L, int64_t row, int64_t vocab_real, int shard_width,
                                               float t, float p, int64_t k, int64_t tg,
                                               float* __restrict__ policy_out, float* __restrict__ ref_out,
                                               float* __restrict__ lse_out,
                                               rlk_support_state* __restrict__ state_out) {
  const RowStart rs = row_start(L.sm, vocab_real, shard_width, t, p, k, tg);
  if (threadIdx.x == 0) {
    ref_out[row] = rs.ref;
    if (lse_out) lse_out[row] = rs.lse;
    write_unsearched(row, rs, policy_out, state_out);
  }
}

// The reference and the policy of a row whose window is complete and holds
// every real token or counts it as -inf, from the exact class masses. All
// kNucWaves wavefronts call it. It returns false, block-uniformly, when the
// row takes the float32 reference instead: a target outside the real columns
// (before any barrier), no finite token or a row maximum beyond the search's
// range (after the row-maximum scan's barrier). Otherwise the wavefronts other
// than 0 return true after the step totals' barrier and wavefront 0 writes
// ref_out, lse_out, policy_out and state_out for the row; bt is the target's
// BF16 pattern.
__device__ __forceinline__ bool exact_row(NucLds& L, int64_t row, int64_t vocab_real, float t, float p, int64_t k,
                                          int64_t tg, uint32_t bt, float* __restrict__ policy_out,
                                          float* __restrict__ ref_out, float* __restrict__ lse_out,
                                          rlk_support_state* __restrict__ state_out) {
  if (tg < 0 || tg >= vocab_real) return false;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const float c = kLog2e / t;  // IEEE float32 division
  // the row maximum, the same in every wavefront: the count's largest pattern
  // when the row holds +0 or a positive token (every token lies in the window
  // here), else the first non-empty class of the scan
  int vm = -32768;
#pragma unroll
  for (int w = 0; w < kNucWaves; ++w) vm = max(vm, L.vmax_w[w]);
  int jtop;
  if (vm > 0) {
    jtop = kNMag - 1 - (vm - static_cast<int>(kMagLo));
  } else if (vm == 0) {
    jtop = kZeroRank;
  } else {
    jtop = window_top_rank(L, lane, wave);
  }
  if (jtop == kNoRank) return false;
  const float m = rank_value(jtop);
  if (!(fabsf(m * c) < kMaxSupportArg)) return false;
  const float R = ref_exponent(m, c);
  const float nr = -R;
  const int sfirst = rank_step(jtop);
  // The steps from s_end on hold no class of nonzero weight: the first step
  // after sfirst whose first (largest) class weighs 0, found by one ballot
  // with lane l testing step l (classes are in decreasing value order).
  const u64 zero_from = __ballot(lane > sfirst && lane < kSteps &&
                                 fmaf(rank_value(step_rank(lane < kSteps ? lane : 0, 0, 0)), c, nr) < -42.0f);
  const int s_end = zero_from ? __builtin_ctzll(zero_from) : kSteps;
  // step totals, in parallel: wavefront w takes steps sfirst + w, + 8, ...
  for (int s = sfirst + wave; s < kSteps; s += kNucWaves) {
    uint32_t tc;
    u64 tm;
    step_total(L, s, s_end, lane, c, nr, tc, tm);
    if (lane == 0) {
      L.st_c[s] = tc;
      L.st_m[s] = tm;
    }
  }
  __syncthreads();
  if (wave != 0) return true;

  // Wavefront 0: lane s holds step s (nothing before sfirst); inclusive
  // prefix sums over the steps.
  const bool live = lane >= sfirst && lane < kSteps;
  const uint32_t sc = live ? L.st_c[lane] : 0u;
  const u64 sm = live ? L.st_m[lane] : 0ull;
  const uint32_t cc = wave_incl_scan<uint32_t>(sc, lane);
  const u64 cm = wave_incl_scan<u64>(sm, lane);
  const uint32_t total_c = lane63(cc);  // the finite tokens
  const u64 z = lane63(cm);             // the row's exact total mass
  uint32_t ninf_n = 0;
  for (int w = 0; w < kNucWaves; ++w) ninf_n += L.red_u32[w][1];

  // top-k boundary by count (the -inf class when the row holds fewer than k
  // finite tokens)
  const bool k_active = (k != -1) && (k < vocab_real);
  int jk = kNoRank;
  uint32_t cnt_k = total_c + ninf_n;
  u64 z_k = z;
  if (k_active && static_cast<uint64_t>(total_c) >= static_cast<uint64_t>(k)) {
    const uint64_t kk = static_cast<uint64_t>(k);
    const int s = __builtin_ctzll(__ballot(static_cast<uint64_t>(cc) >= kk));  // first step reaching k
    const uint32_t carry_c = readlane_u32(cc - sc, s);
    const u64 carry_m = readlane_u64(cm - sm, s);
    StepRound Q;
    step_round(L, s, c, nr, Q);
    int hit_e = -1;
#pragma unroll
    for (int e = 3; e >= 0; --e) {
      const uint64_t cum = carry_c + Q.cum_c[e];
      if (cum >= kk && cum - Q.cnt[e] < kk) hit_e = e;
    }
    const u64 ball = __ballot(hit_e >= 0);  // nonzero: the step holds the k-th token
    const int hl = __builtin_ctzll(ball);
    const int he = __builtin_amdgcn_readlane(hit_e, hl);
    uint32_t hc = 0;
    u64 hm = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e == he) {
        hc = Q.cum_c[e];
        hm = Q.cum_m[e];
      }
    jk = step_rank(s, hl, he);
    cnt_k = carry_c + readlane_u32(hc, hl);
    z_k = carry_m + readlane_u64(hm, hl);
  }

  // top-p boundary by mass inside the top-k set: the first class whose
  // cumulative mass reaches P = ceil(p * z_k) <= z_k. Its step is the first
  // whose inclusive mass reaches P, which is not after jk's step.
  int kappa = jk;
  uint32_t cnt_s = cnt_k;
  u64 z_s = z_k;
  if (p < 1.0f) {
    const u64 P = ceil_mul(p, z_k);
    const int s = __builtin_ctzll(__ballot(cm >= P));
    const uint32_t carry_c = readlane_u32(cc - sc, s);
    const u64 carry_m = readlane_u64(cm - sm, s);
    StepRound Q;
    step_round(L, s, c, nr, Q);
    int e_p = -1;
#pragma unroll
    for (int e = 3; e >= 0; --e) {
      const u64 cum = carry_m + Q.cum_m[e];
      const int r = step_rank(s, lane, e);
      const bool inside = r >= 0 && r <= jk;
      if (inside && cum >= P && cum - Q.mass[e] < P) e_p = e;
    }
    const u64 ball = __ballot(e_p >= 0);  // nonzero: the crossing lies in this step
    const int hl = __builtin_ctzll(ball);
    const int he = __builtin_amdgcn_readlane(e_p, hl);
    uint32_t hc = 0;
    u64 hm = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e == he) {
        hc = Q.cum_c[e];
        hm = Q.cum_m[e];
      }
    kappa = step_rank(s, hl, he);
    cnt_s = carry_c + readlane_u32(hc, hl);
    z_s = carry_m + readlane_u64(hm, hl);
  }

  if (lane == 0) {
    // the reference: lse = (R + log2(Z) - 40) * ln 2, in float64 as for the shard merge
    const double lse = (static_cast<double>(R) + (log2(static_cast<double>(z)) - 40.0)) * kLn2;
    const float zt = __uint_as_float(bt << 16) / t;  // IEEE float32 division
    RowStart rs;
    rs.ref = static_cast<float>(static_cast<double>(zt) - lse);
    rs.lse = static_cast<float>(lse);
    rs.bt = bt;
    rs.status = 0;
    ref_out[row] = rs.ref;
    if (lse_out) lse_out[row] = rs.lse;
    write_policy(row, vocab_real, true, kappa, cnt_s, z_s, R, true, rs, t, policy_out, state_out);
  }
  return true;
}

// ---------------------------------------------------------------------------
// Whole-row driver for all threads of the block, from the row's 8 float32
// shard summaries in L.sm, the window and the count totals of the streaming
// pass. A row that needs a search and whose real tokens all lie
// in the window (or are -inf) takes the exact path; the other searched rows
// take the float32 reference, with no support when the row maximum is beyond
// the search's range, or with the general path's support when a token lies
// outside the window. Writes ref_out[row], policy_out[row] and, when given,
// lse_out[row] and state_out[row].
// ---------------------------------------------------------------------------
__device__ __forceinline__ void nucleus_row(NucLds& L, const uint16_t* __restrict__ rowp, int64_t row,
                                            int64_t vocab_real, int shard_width, float t, float p, int64_t k,
                                            int64_t tg, float* __restrict__ policy_out,
                                            float* __restrict__ ref_out, float* __restrict__ lse_out,
                                            rlk_support_state* __restrict__ state_out) {
  const int tid = threadIdx.x;
  RowStart rs;
  rs.ref = NAN;
  rs.lse = NAN;
  rs.bt = 0;
  rs.status = -2;
  if (tid == 0) {
    rs = row_start(L.sm, vocab_real, shard_width, t, p, k, tg);
    L.search = (rs.status == 0);
    L.tbits = rs.bt;
    L.k_active = (k != -1) && (k < vocab_real);
    L.p_active = (p < 1.0f);
    L.k = k;
    L.p = p;
    L.c = kLog2e / t;
    if (rs.status != 0) {
      ref_out[row] = rs.ref;
      if (lse_out) lse_out[row] = rs.lse;
      write_unsearched(row, rs, policy_out, state_out);
    }
  }
  __syncthreads();
  if (!L.search) return;

  bool odd = false;  // block-uniform: a real token outside the window
  for (int w = 0; w < kNucWaves; ++w) odd |= (L.red_flag[w] != 0);
  if (!odd) {
    if (exact_row(L, row, vocab_real, t, p, k, tg, L.tbits, policy_out, ref_out, lse_out, state_out)) return;
    // the row maximum lies beyond the search's range: no support
    if (tid == 0) {
      ref_out[row] = rs.ref;
      if (lse_out) lse_out[row] = rs.lse;
      RowStart none = rs;
      none.status = -1;
      write_unsearched(row, none, policy_out, state_out);
    }
    return;
  }
  if (tid == 0) {
    ref_out[row] = rs.ref;
    if (lse_out) lse_out[row] = rs.lse;
  }
  __syncthreads();  // the flags above are read before the general path reuses the block scratch
  support_general(L, rowp, vocab_real);
  if (tid == 0)
    write_policy(row, vocab_real, false, L.kappa, L.cnt_s, L.z_s, L.R, L.in_range != 0, rs, t, policy_out, state_out);
}

}  // namespace rlk
