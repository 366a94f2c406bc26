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
// Fast path: every token is counted (LDS u32 atomics) in a window of classes:
// the BF16 values of magnitude in [2^-24, 65536) of either sign, interleaved
// by magnitude (slot 2*(m - m_lo) + sign, m the 15-bit magnitude pattern),
// plus one class for +-0; -inf tokens are counted apart (mass 0). The slots of
// two tokens come from three packed 16-bit instructions, and one maximum over
// a vector's eight slots tells whether all of them lie in the window. Classes
// are visited in value order (positive slots from the largest magnitude down,
// the zero class, negative slots from the smallest magnitude up). With groups == 1 the
// shard-waves count while they stream the row for the reference logprob, so
// the support costs no extra pass; otherwise one pass builds it. The row
// maximum is the first non-empty class, class masses are count * weight, and
// the thresholds come from prefix sums over the classes, computed by one
// wavefront while the rest of the workgroup has finished (with groups == 1 a
// second wavefront merges the shard summaries meanwhile). When top-k is off,
// the top-p threshold ceil(p * Z) is first bracketed from the float shard
// sums, so the total Z is summed only when the bracket cannot decide; a scan
// that runs past three steps skips ahead by four-step mass totals.
// General path, for rows with a token outside the window (a nonzero value of
// magnitude below 2^-24, or 65536 and beyond): an exact-maximum pass, then a
// 4096-bin histogram of (count, mass) over key >> 4, then the 16 keys of each
// boundary bin, each from another pass over the row. Both paths produce the
// same integers and therefore the same output bytes.
#pragma once

#include "logp_device.hpp"
#include "rlk_logp.h"

namespace rlk {

constexpr int kNucThreads = 512;
constexpr int kNucWaves = kNucThreads / kWave;
constexpr int kBinsA = 4096;
constexpr int kSub = 16;
// The window: magnitudes kMagLo .. kMagLo + kNMag - 1 (2^-24 <= |x| < 65536)
// of both signs, interleaved, then the zero class. 40 KB of counts: three rows
// per CU with the general path's histogram in the same LDS.
constexpr uint32_t kMagLo = 0x3380u;               // magnitude pattern of 2^-24
constexpr int kNMag = 5120;                        // 40 binades of 128 BF16 values
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
// it gets no support (policy NaN, status -1); its reference is unaffected.
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
// nonzero magnitudes below 2^-24, magnitudes of 65536 and beyond).
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
  // the row merge, handed from wavefront 1 to wavefront 0 (RowStart)
  float rs_ref;
  float rs_lse;
  uint32_t rs_bt;
  int rs_status;
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

// Nonzero unless all 8 slots of a vector (4 words of slot pairs) are below
// kWin: the packed maximum of the 8, then a saturating subtraction of kWin - 1.
__device__ __forceinline__ uint32_t slots_outside(const uint32_t (&sl)[4]) {
  uint32_t e0, e1, e, out;
  asm("v_pk_max_u16 %[e0], %[s0], %[s1]\n\t"
      "v_pk_max_u16 %[e1], %[s2], %[s3]\n\t"
      "v_pk_max_u16 %[e], %[e0], %[e1]\n\t"
      "v_pk_sub_u16 %[out], %[e], %[top] clamp"
      : [e0] "=&v"(e0), [e1] "=&v"(e1), [e] "=&v"(e), [out] "=&v"(out)
      : [s0] "v"(sl[0]), [s1] "v"(sl[1]), [s2] "v"(sl[2]), [s3] "v"(sl[3]), [top] "v"(0x27FF27FFu));
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

  // One token: its exact slot (zero class included), or the outside tally.
  __device__ __forceinline__ void one(uint32_t b) {
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

  // v: one vector of 8 BF16 columns as loaded; x: their float32 widenings;
  // nvalid of them are real (the first nvalid).
  __device__ __forceinline__ void operator()(const u32x4& v, const float (&x)[8], int nvalid) {
    if (nvalid == 8) {
      full(v);
    } else {
      for (int e = 0; e < nvalid; ++e) one(__float_as_uint(x[e]) >> 16);
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
  for (int i = threadIdx.x; i < kWinWords / 2; i += kNucThreads) L.u.win_pairs[i] = 0ull;
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

// ---------------------------------------------------------------------------
// Fast path, in one wavefront (no block barriers), for a row whose every real
// token is in the window or is -inf (the hook totals say so). The row maximum
// is the first non-empty class, R = ceil(fl32(M*c)), and a class weighs
// count * floor(2^(x*c - R) * 2^40): exactly the integers the general path
// sums per token. Scans in value order find the top-k boundary (count >= k)
// and then the top-p boundary (cumulative mass >= ceil(p * Z_k), an exact
// integer test). The classes are visited in steps of 256 ranks: the positive
// slots in 20 steps, the zero class alone, the negative slots in 20 steps. In
// a step lane l holds ranks 4l .. 4l+3 (two 16-byte LDS reads cover the 8
// interleaved slots of its 4 magnitudes); prefix sums come from a lane-local
// scan plus a DPP scan of the lane totals, and a crossing is located with a
// ballot. Every value it returns is wave-uniform.
// ---------------------------------------------------------------------------
struct FastSupport {
  float R;
  int kappa;       // rank of the last kept class, or kNoRank for the -inf class
  uint32_t cnt_s;  // tokens in the support
  u64 z_s;         // support mass (2^-40 units relative to 2^R)
  bool in_range;   // the row maximum lies in the search's range (kMaxSupportArg)
};

constexpr int kStepRanks = 4 * kWave;           // 256 ranks per step
constexpr int kPosSteps = kNMag / kStepRanks;   // 20
constexpr int kZeroStep = kPosSteps;
constexpr int kSteps = 2 * kPosSteps + 1;
static_assert(kNMag % kStepRanks == 0, "steps cover whole magnitude ranges");

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

// One step: per-class counts and masses, and the inclusive cumulative count
// and mass of each class counted from the step's first class (lane-local
// prefix plus the exclusive DPP scan of the lanes). Returns the step's totals
// through rc / rm, and false (wave-uniform, with zero totals and Q left
// unset) when all its classes are empty.
struct StepRound {
  uint32_t cnt[4];
  u64 mass[4];
  uint32_t cum_c[4];
  u64 cum_m[4];
};

__device__ __forceinline__ bool step_round(const NucLds& L, int s, float c, float nr, StepRound& Q, uint32_t& rc,
                                           u64& rm) {
  const int lane = threadIdx.x & (kWave - 1);
  step_counts(L, s, lane, Q.cnt);
  if (__ballot((Q.cnt[0] | Q.cnt[1] | Q.cnt[2] | Q.cnt[3]) != 0u) == 0ull) {  // wave-uniform
    rc = 0u;
    rm = 0ull;
    return false;
  }
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
  const uint32_t ic = wave_incl_scan<uint32_t>(pc, lane);
  const u64 im = wave_incl_scan<u64>(pm, lane);
  const uint32_t ec = ic - pc;
  const u64 em = im - pm;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    Q.cum_c[e] += ec;
    Q.cum_m[e] += em;
  }
  rc = readlane_u32(ic, kWave - 1);
  rm = readlane_u64(im, kWave - 1);
  return true;
}

constexpr int kBatch = 4;       // steps whose LDS reads a scan issues together
constexpr int kRoundSteps = 3;  // steps a top-p scan takes class by class before it skips ahead

// Count and mass of the classes that `lane` holds in steps s .. s + kBatch - 1
// (steps at or past s_end count zero), summed lane-locally; the LDS reads of
// the kBatch steps are issued before any of them is used.
__device__ __forceinline__ void batch_lane_sums(const NucLds& L, int s, int s_end, int lane, float c, float nr,
                                                uint32_t (&pc)[kBatch], u64 (&pm)[kBatch]) {
  uint32_t cn[kBatch][4];
#pragma unroll
  for (int b = 0; b < kBatch; ++b) {
    if (s + b < s_end) {
      step_counts(L, s + b, lane, cn[b]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) cn[b][e] = 0u;
    }
  }
#pragma unroll
  for (int b = 0; b < kBatch; ++b) {
    uint32_t sum_hi = 0u;  // sum of count * hi: below 2^24 * 256 over a row
    u64 sum_lo = 0ull;
    pc[b] = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t hi, lo;
      weight_parts(step_bits(s + b, lane, e), c, nr, hi, lo);
      sum_hi += static_cast<uint32_t>(__umul24(cn[b][e], hi));
      sum_lo += static_cast<u64>(cn[b][e]) * lo;
      pc[b] += cn[b][e];
    }
    pm[b] = (static_cast<u64>(sum_hi) << 32) + sum_lo;
  }
}

__device__ __forceinline__ FastSupport support_fast_wave(const NucLds& L, int64_t vocab_real, int shard_width,
                                                         bool k_active, int64_t k_in, bool p_active, float p,
                                                         float c) {
  const int lane = threadIdx.x & (kWave - 1);
  FastSupport out;
  uint32_t ninf_n = 0;
  for (int w = 0; w < kNucWaves; ++w) ninf_n += L.red_u32[w][1];
  const uint32_t total_c = static_cast<uint32_t>(vocab_real) - ninf_n;

  // the row maximum: the first non-empty class, at or above the class of the
  // largest shard-summary m (each is a token of the row, so it lies in the
  // window); kBatch steps per iteration, their LDS reads issued together
  float mb = -INFINITY;
#pragma unroll
  for (int sh = 0; sh < kShards; ++sh) mb = fmaxf(mb, L.sm[sh].m);
  int jtop = kNoRank;
  if (mb > -INFINITY) {
    const uint32_t sl = window_slot(__float_as_uint(mb) >> 16);
    const int sb = (sl == kSlotOut) ? kSteps - 1 : rank_step(slot_rank(sl));
    for (int s0 = 0; s0 <= sb; s0 += kBatch) {
      uint32_t cn[kBatch][4];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (s0 + b <= sb) {
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
      if (hit >= 0) {
        int j = kNoRank;
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
          if (b == hit) {
#pragma unroll
            for (int e = 3; e >= 0; --e)
              if (cn[b][e]) j = step_rank(s0 + b, lane, e);
          }
        jtop = wave_min(j);
        break;
      }
    }
  }
  out.kappa = kNoRank;
  out.cnt_s = total_c + ninf_n;
  out.z_s = 0;
  out.R = 0.0f;
  out.in_range = true;
  if (jtop == kNoRank) return out;  // no finite token: not reached on a searched row
  const float m = rank_value(jtop);
  const float R = ref_exponent(m, c);
  const float nr = -R;
  out.R = R;
  out.in_range = fabsf(m * c) < kMaxSupportArg;  // wave-uniform
  if (!out.in_range) return out;
  const int sfirst = rank_step(jtop);

  // exact mass of the classes from step s_start on: lane-local sums over the
  // steps, one wave reduction. Every class with a nonzero weight lies before
  // the first step whose first class is below 2^-42 (the classes are in
  // decreasing value order).
  // The steps from s_end on hold no class of nonzero weight: the first step
  // after sfirst whose first (largest) class weighs 0, found by one ballot
  // with lane l testing step l.
  const u64 zero_from = __ballot(lane > sfirst && lane < kSteps &&
                                 fmaf(rank_value(step_rank(lane < kSteps ? lane : 0, 0, 0)), c, nr) < -42.0f);
  const int s_end = zero_from ? __builtin_ctzll(zero_from) : kSteps;
  auto exact_mass_from = [&](int s_start) -> u64 {
    u64 acc = 0;
    for (int s = s_start; s < s_end; s += kBatch) {
      uint32_t pc[kBatch];
      u64 pm[kBatch];
      batch_lane_sums(L, s, s_end, lane, c, nr, pc, pm);
#pragma unroll
      for (int b = 0; b < kBatch; ++b) acc += pm[b];
    }
    return wave_total<u64>(acc);
  };

  // top-k boundary by count (the -inf class when the window holds fewer than k)
  int jk = kNoRank;
  uint32_t cnt_k = total_c + ninf_n;
  u64 z_k = 0;
  bool z_k_known = false;  // otherwise z_k is the row's total mass, not yet summed
  if (k_active && static_cast<uint64_t>(total_c) >= static_cast<uint64_t>(k_in)) {
    const uint64_t k = static_cast<uint64_t>(k_in);
    uint32_t carry_c = 0;
    u64 carry_m = 0;
    for (int s = sfirst; s < kSteps; ++s) {
      StepRound Q;
      uint32_t rc;
      u64 rm;
      if (!step_round(L, s, c, nr, Q, rc, rm)) continue;  // no token in this step
      int hit_e = -1;
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        const uint64_t cum = carry_c + Q.cum_c[e];
        if (cum >= k && cum - Q.cnt[e] < k) hit_e = e;
      }
      const u64 ball = __ballot(hit_e >= 0);
      if (ball) {  // wave-uniform
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
        z_k_known = true;
        break;
      }
      carry_c += rc;
      carry_m += rm;
    }
  }

  // top-p boundary by mass inside the top-k set: the first class whose
  // cumulative mass reaches P = ceil(p * z_k). Scanning for thresholds
  // p_lo <= P <= p_hi finds classes j_lo <= j* <= j_hi (cumulative masses only
  // grow), so j_lo == j_hi decides j* exactly. A scan runs from a position
  // (a step and the count and mass of every class before it) and leaves the
  // position after the step where it found p_hi's crossing (or at the end of
  // the classes); `lo_pos` is the start of the step holding j_lo.
  struct Hit {
    int j;
    uint32_t cnt;
    u64 mass;
  };
  struct ScanPos {
    int s;
    uint32_t c;
    u64 m;
  };
  auto scan_p = [&](ScanPos& pos, u64 p_lo, u64 p_hi, Hit& lo, ScanPos& lo_pos, int& j_hi) {
    lo.j = -1;
    j_hi = -1;
    for (int n_round = 0; pos.s < kSteps; ++pos.s, ++n_round) {
      if (n_round >= kRoundSteps) {
        // skip ahead: the totals of the next kBatch steps carry the position
        // up to the step where the pending threshold is crossed (cumulative
        // masses only grow, so no class before it can be the crossing)
        const u64 thr = (lo.j < 0) ? p_lo : p_hi;
        uint32_t pc[kBatch];
        u64 pm[kBatch];
        batch_lane_sums(L, pos.s, s_end, lane, c, nr, pc, pm);
        const u64 tm_all = wave_total<u64>((pm[0] + pm[1]) + (pm[2] + pm[3]));
        if (pos.m + tm_all < thr) {  // wave-uniform: no crossing in the batch
          pos.m += tm_all;
          pos.c += wave_total<uint32_t>((pc[0] + pc[1]) + (pc[2] + pc[3]));
          pos.s += kBatch - 1;  // the loop's increment moves past the batch
          if (pos.s + 1 >= s_end) pos.s = kSteps - 1;  // no weight below: the end of the classes
          continue;
        }
        // the crossing lies in the batch: the steps before it by their totals
        u64 run = pos.m;
        uint32_t runc = 0u;
        int skip = kBatch - 1;
#pragma unroll
        for (int b = 0; b < kBatch - 1; ++b) {
          if (skip == kBatch - 1) {
            const u64 tm = wave_total<u64>(pm[b]);
            if (run + tm >= thr) {
              skip = b;
            } else {
              run += tm;
              runc += pc[b];
            }
          }
        }
        pos.m = run;
        pos.c += wave_total<uint32_t>(runc);
        pos.s += skip;  // the step holding the crossing, scanned class by class below
      }
      StepRound Q;
      uint32_t rc;
      u64 rm;
      if (!step_round(L, pos.s, c, nr, Q, rc, rm)) continue;  // no token in this step
      int e_lo = -1, e_hi = -1;
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        const u64 cum = pos.m + Q.cum_m[e];
        const int r = step_rank(pos.s, lane, e);
        const bool inside = r >= 0 && r <= jk;
        if (inside && cum >= p_lo && cum - Q.mass[e] < p_lo) e_lo = e;
        if (inside && cum >= p_hi && cum - Q.mass[e] < p_hi) e_hi = e;
      }
      const u64 b_lo = __ballot(e_lo >= 0);
      if (b_lo && lo.j < 0) {  // wave-uniform
        const int hl = __builtin_ctzll(b_lo);
        const int he = __builtin_amdgcn_readlane(e_lo, hl);
        uint32_t hc = 0;
        u64 hm = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e == he) {
            hc = Q.cum_c[e];
            hm = Q.cum_m[e];
          }
        lo.j = step_rank(pos.s, hl, he);
        lo.cnt = pos.c + readlane_u32(hc, hl);
        lo.mass = pos.m + readlane_u64(hm, hl);
        lo_pos = pos;
      }
      pos.c += rc;
      pos.m += rm;
      const u64 b_hi = __ballot(e_hi >= 0);
      if (b_hi) {  // wave-uniform
        const int hl = __builtin_ctzll(b_hi);
        j_hi = step_rank(pos.s, hl, __builtin_amdgcn_readlane(e_hi, hl));
        ++pos.s;
        break;
      }
    }
  };

  int kappa = jk;
  uint32_t cnt_s = cnt_k;
  u64 z_s = z_k;
  if (p_active) {
    Hit lo;
    ScanPos lo_pos = {sfirst, 0u, 0ull};
    ScanPos pos = {sfirst, 0u, 0ull};
    int j_hi = -1;
    bool decided = false;
    if (!z_k_known) {
      // The shard summaries bound the total. Each l_s sums positive float32
      // terms 2^(x*c - r_s) through at most `depth` roundings (a lane's
      // vectors plus a partial one, 3 pairwise levels, 6 butterfly levels):
      // relative error <= depth * 2^-24. A term and the token's integer
      // weight floor(2^(x*c - R) * 2^40) differ by the rounding of their
      // exponent arguments, by v_exp_f32 (about 2^-23 each), by the floor
      // (under one unit per token on a total of at least 2^39 units) and by
      // terms whose weight floors to 0 (under 1/4 unit each). The arguments:
      // x*c - r_s is below D_s + 1 (D_s = R - r_s >= 0), and the term of the
      // maximum of the chunk that fixed r_s makes l_s >= 1/2, so the terms
      // with x*c - r_s >= -31 are rounded by at most half an ulp of
      // max(31, D_s + 1) and all the others together move l_s by under 2^-30
      // relative; likewise x*c - R lies in [-42, 0] where a weight is nonzero,
      // rounded by at most 2^-20 (half an ulp of 31) above -31, the rest under
      // 2^-30 relative. A relative argument error d changes 2^arg by d*ln 2 <
      // d. The bracket takes twice the sum.
      const int depth = (shard_width / 8 + kWave) / kWave + 1 + 3 + 6;
      float dmax = 0.0f;
#pragma unroll
      for (int sh = 0; sh < kShards; ++sh)
        if (L.sm[sh].l > 0.0f) dmax = fmaxf(dmax, R - L.sm[sh].r);
      const double karg = fmax(31.0, static_cast<double>(dmax) + 1.0);
      const double half_ulp = ldexp(1.0, ilogb(karg) - 24);
      const double eps = 2.0 * (static_cast<double>(depth) * 0x1p-24 + half_ulp + 0x1p-20 + 0x1p-22 + 0x1p-30 +
                                1.25 * static_cast<double>(vocab_real) * 0x1p-39);
      double zf = 0.0;
#pragma unroll
      for (int sh = 0; sh < kShards; ++sh) {
        const float l = L.sm[sh].l;
        if (l > 0.0f) zf += ldexp(static_cast<double>(l), static_cast<int>(L.sm[sh].r - R) + 40);
      }
      const u64 z_lo = static_cast<u64>(zf * (1.0 - eps));
      const u64 z_hi = static_cast<u64>(zf * (1.0 + eps)) + 1ull;
      ScanPos lo_pos_b = lo_pos;
      scan_p(pos, ceil_mul(p, z_lo), ceil_mul(p, z_hi), lo, lo_pos_b, j_hi);
      decided = (lo.j >= 0) && (lo.j == j_hi);
      if (!decided) {
        // the exact total: the scanned classes' mass plus the mass below them
        z_k = pos.m + exact_mass_from(pos.s);
        z_k_known = true;
        // P >= ceil(p * z_lo), so the exact crossing is not above j_lo: the
        // exact scan restarts at the step holding j_lo
        pos = (lo.j >= 0) ? lo_pos_b : ScanPos{sfirst, 0u, 0ull};
      }
    }
    if (!decided) {
      const u64 P = ceil_mul(p, z_k);
      scan_p(pos, P, P, lo, lo_pos, j_hi);
    }
    kappa = lo.j;
    cnt_s = lo.cnt;
    z_s = lo.mass;
  }
  // (top-p off and top-k keeping every finite token: the support is the whole
  // vocabulary, whose policy output is the reference output; z_s is unused)
  out.kappa = kappa;
  out.cnt_s = cnt_s;
  out.z_s = z_s;
  return out;
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

// Whole row in wavefront 0 alone, for a row whose window is complete (every
// real token in the window or -inf) or that needs no search: no block
// barriers, so the other wavefronts of the workgroup may already have ended.
// Every lane computes the same merge; lane 0 writes.
__device__ __forceinline__ void nucleus_row_wave(const NucLds& L, int64_t row, int64_t vocab_real, int shard_width,
                                                 float t, float p, int64_t k, int64_t tg,
                                                 float* __restrict__ policy_out, float* __restrict__ ref_out,
                                                 float* __restrict__ lse_out,
                                                 rlk_support_state* __restrict__ state_out) {
  const bool lead = (threadIdx.x == 0);
  const RowStart rs = row_start(L.sm, vocab_real, shard_width, t, p, k, tg);
  if (lead) {
    ref_out[row] = rs.ref;
    if (lse_out) lse_out[row] = rs.lse;
  }
  if (rs.status != 0) {
    if (lead) write_unsearched(row, rs, policy_out, state_out);
    return;
  }
  const bool k_active = (k != -1) && (k < vocab_real);
  const bool p_active = (p < 1.0f);
  const FastSupport fs = support_fast_wave(L, vocab_real, shard_width, k_active, k, p_active, p, kLog2e / t);
  if (lead) write_policy(row, vocab_real, true, fs.kappa, fs.cnt_s, fs.z_s, fs.R, fs.in_range, rs, t, policy_out,
                 state_out);
}

// A searched row whose window is complete, in two wavefronts: wavefront 1
// merges the summaries and writes the reference outputs while wavefront 0
// runs the support search, then wavefront 0 writes the policy outputs. The
// other wavefronts of the workgroup have ended, and a barrier waits only for
// the wavefronts still running.
__device__ __forceinline__ void nucleus_row_pair(NucLds& L, int wave, int64_t row, int64_t vocab_real,
                                                 int shard_width, float t, float p, int64_t k, int64_t tg,
                                                 float* __restrict__ policy_out, float* __restrict__ ref_out,
                                                 float* __restrict__ lse_out,
                                                 rlk_support_state* __restrict__ state_out) {
  const bool lead = (threadIdx.x & (kWave - 1)) == 0;
  FastSupport fs;
  if (wave == 1) {
    const RowStart rs = row_start(L.sm, vocab_real, shard_width, t, p, k, tg);
    if (lead) {
      ref_out[row] = rs.ref;
      if (lse_out) lse_out[row] = rs.lse;
      L.rs_ref = rs.ref;
      L.rs_lse = rs.lse;
      L.rs_bt = rs.bt;
      L.rs_status = rs.status;
    }
  } else {
    const bool k_active = (k != -1) && (k < vocab_real);
    const bool p_active = (p < 1.0f);
    fs = support_fast_wave(L, vocab_real, shard_width, k_active, k, p_active, p, kLog2e / t);
  }
  __syncthreads();
  if (wave == 0 && lead) {
    RowStart rs;
    rs.ref = L.rs_ref;
    rs.lse = L.rs_lse;
    rs.bt = L.rs_bt;
    rs.status = L.rs_status;
    if (rs.status != 0)
      write_unsearched(row, rs, policy_out, state_out);
    else
      write_policy(row, vocab_real, true, fs.kappa, fs.cnt_s, fs.z_s, fs.R, fs.in_range, rs, t, policy_out,
                 state_out);
  }
}

// ---------------------------------------------------------------------------
// Whole-row driver for all threads of the block: L.sm must hold the row's 8
// shard summaries; when `window_built` the window and the hook totals are
// already filled (the streaming pass counted the row). After the window is
// complete, a row whose tokens all lie in it continues in wavefront 0 alone
// (support_fast_wave; the other wavefronts return); other rows take the
// general path with the whole block. Writes ref_out[row], policy_out[row] and,
// when given, lse_out[row] and state_out[row].
// ---------------------------------------------------------------------------
__device__ __forceinline__ void nucleus_row(NucLds& L, const uint16_t* __restrict__ rowp, int64_t row,
                                            int64_t vocab_real, int shard_width, float t, float p, int64_t k,
                                            int64_t tg, bool window_built, float* __restrict__ policy_out,
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
    ref_out[row] = rs.ref;
    if (lse_out) lse_out[row] = rs.lse;
    L.search = (rs.status == 0);
    if (rs.status == 0) {
      L.k_active = (k != -1) && (k < vocab_real);
      L.p_active = (p < 1.0f);
      L.k = k;
      L.p = p;
      L.c = kLog2e / t;
    } else {
      write_unsearched(row, rs, policy_out, state_out);
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
  bool odd = false;  // block-uniform: a real token outside the window
  for (int w = 0; w < kNucWaves; ++w) odd |= (L.red_flag[w] != 0);
  if (!odd) {
    if (tid >= kWave) return;
    const FastSupport fs =
        support_fast_wave(L, vocab_real, shard_width, L.k_active != 0, L.k, L.p_active != 0, L.p, L.c);
    if (tid == 0) write_policy(row, vocab_real, true, fs.kappa, fs.cnt_s, fs.z_s, fs.R, fs.in_range, rs, t, policy_out,
                 state_out);
    return;
  }
  __syncthreads();  // the flags above are read before the general path reuses the block scratch
  support_general(L, rowp, vocab_real);
  if (tid == 0)
    write_policy(row, vocab_real, false, L.kappa, L.cnt_s, L.z_s, L.R, L.in_range != 0, rs, t, policy_out, state_out);
}

}  // namespace rlk
