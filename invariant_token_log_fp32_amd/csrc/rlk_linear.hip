// LM-head linear layer and fused linear + token logprob ("linear-logp") for
// gfx950, and the C-ABI declared in include/rlk_linear.h.
//
// Passages: RL-Kernel page "Reproduce and profile the Qwen3-8B TP4/CP2
// experiment", section "Capture logs, status, and validation evidence" (the
// run log is audited for the linear-logp backend), and page "Configurable H100
// consistency runs", sampling and mode/KL paragraphs (BF16 model logits,
// float32 temperature scaling, full-vocabulary reference logprob).
//
// Kernels:
//   k_linear<kLogp>  one 256 x 256 tile of logits per step of a grid-stride
//                    loop over tiles, in XCD-aware groups of 4 x 8 tiles
//                    that share operand panels in L2; 4 waves (one per SIMD),
//                    each 128 x 128 as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16
//                    (the largest wave tile the 512 registers hold, so the
//                    fewest LDS reads per multiply-add; the 32 x 32 blocks
//                    need 8 fragments per K step of 16, which leaves registers
//                    for a second set in flight and the staged panels).
//                    K runs in 64-wide stages (four MFMA steps of 16) through
//                    double-buffered LDS. Panels go from global memory to LDS
//                    directly (16-byte buffer loads into LDS: no registers,
//                    no LDS store instructions); the loads' range check
//                    returns zeros for rows past the operand's end. A load
//                    instruction fills 1 KB of LDS in lane order, so rows are
//                    128 bytes with the 16-byte chunks of row r permuted by
//                    an XOR with swz(r) (no bank conflicts for the fragment
//                    reads). Each step's multiplies run with the LDS reads of
//                    the next step's fragments; step 3 also issues the loads
//                    of the stage after next into the buffer just finished
//                    with; one barrier per stage, before step 3, after the
//                    next stage's loads have landed.
//                    Epilogue: the fp32 accumulators are rounded to BF16 into
//                    an LDS tile, then either stored (rlk_linear) or reduced
//                    per row to a 16-byte summary of the tile's 128 columns
//                    (rlk_linear_logp) for each 128 columns: integer reference
//                    exponent r from their exact maximum and l = sum of
//                    2^(x*c - r) in a fixed order; greedy rows keep the
//                    maximum and its lowest column.
//   k_lin_merge      one wave per row: the row's 128-column summaries merged
//                    in column order (fp64), then the target's logprob.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "logp_device.hpp"
#include "rlk_linear.h"
#include "rlk_logp.h"

namespace rlk_lin {

using rlk::ShardSummary;
using rlk::u32x4;

constexpr int BM = 256;                 // rows of a workgroup tile
constexpr int BN = 256;                 // vocabulary columns of a workgroup tile
constexpr int BK = 64;                  // K per LDS stage
constexpr int SN = 128;                 // columns per summary (nests in the canonical shards)
constexpr int kThreads = 256;           // 4 waves, 2 x 2, each 128 x 128 (one per SIMD)
constexpr int kWaveM = 128;
constexpr int kWaveN = 128;
constexpr int kMB = kWaveM / 32;        // 32 x 32 MFMA blocks per wave
constexpr int kNB = kWaveN / 32;
constexpr int kSteps = BK / 16;         // MFMA K steps per stage
constexpr int kLdsRow = BK;             // bf16 per LDS row: 128 bytes, chunks permuted (swz)
constexpr int kStage = BM * kLdsRow;    // bf16 per operand per stage (BM == BN)
constexpr int kChunks = BM * BK / 8 / kThreads;  // 16-byte loads per thread per operand per stage
constexpr int kOutRow = BN + 8;         // bf16 per row of the epilogue tile: 528 bytes
constexpr int64_t kMaxGrid = int64_t(1) << 20;
// XCD-aware order: workgroup b runs on XCD b % 8; each XCD takes groups of
// kGM x kGN tiles (one per CU of the XCD), so the 32 workgroups of a group
// stream the same 4 hidden-state panels and 8 vocabulary panels through that
// XCD's L2, stage by stage.
constexpr int kXcds = 8;
constexpr int kGM = 4;
constexpr int kGN = 8;
constexpr int64_t kMaxRows = int64_t(1) << 22;
constexpr int64_t kMaxLd = int64_t(1) << 21;  // row strides: a panel's byte offsets fit 31 bits
constexpr int64_t kMaxVocab = int64_t(1) << 30;
constexpr int kMaxD = 65536;

static_assert(BM == BN, "one LDS stage shape for both operands");
constexpr int kSmem = (4 * kStage > BM * kOutRow) ? 4 * kStage : BM * kOutRow;  // bf16: stages, or the epilogue tile
static_assert(BN % SN == 0, "whole summaries per tile");
static_assert((BM / kWaveM) * (BN / kWaveN) * 64 == kThreads, "one wave per wave tile");
static_assert(kChunks == 8, "the interleaving below issues 8 panel loads per operand, thread and stage");
static_assert(kLdsRow == 64 && kThreads == 256, "the load-to-LDS mapping assumes 8 chunks per row, 4 waves");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef f32x16 Acc;  // accumulator of one 32 x 32 block: 16 floats per lane

struct Geo {
  const uint16_t* __restrict__ h;
  const uint16_t* __restrict__ w;
  int64_t ldh;
  int64_t ldw;
  int64_t n_rows;
  int64_t vocab_real;
  int64_t vocab_padded;
  int d;
  int m_tiles;
  int64_t col_base; // first (global) vocabulary column of this launch
  int64_t col_end;  // end of its columns (multiple of SN, at most vocab_padded)
  int64_t w_end;    // end of the columns with a projection row: min(col_end, vocab_real)
  int64_t n_tiles;  // workgroup tiles along the vocabulary
  int64_t n_sum;    // summaries per row in this launch (SN columns each)
  int64_t m_groups; // tile groups along the rows (kGM tiles each)
  int64_t n_groups; // tile groups along the vocabulary (kGN tiles each)
};

// Tile of virtual workgroup v, or false when v has no tile.
__device__ __forceinline__ bool tile_of(const Geo& g, int64_t v, int64_t& m_t, int64_t& n_t) {
  const int64_t xcd = v % kXcds;
  const int64_t slot = v / kXcds;
  const int64_t k = (slot / (kGM * kGN)) * kXcds + xcd;  // group id
  const int64_t local = slot % (kGM * kGN);
  if (k >= g.m_groups * g.n_groups) return false;
  m_t = (k % g.m_groups) * kGM + local % kGM;
  n_t = (k / g.m_groups) * kGN + local / kGM;
  return m_t < g.m_tiles && n_t < g.n_tiles;
}

// Chunk permutation of the LDS rows: chunk c (8 bf16) of row r sits in slot
// c ^ swz(r). For the fragment reads (lane l: row l%32 of a 32-row block,
// chunk 2kk + l/32) the 16 rows read together at one chunk land in 16
// different 16-byte bank groups, and the rows 0-7 of lanes 0-7 and 32-39 (two
// neighbouring chunks) in disjoint ones.
__host__ __device__ __forceinline__ constexpr int swz(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }

// The operand panels of a tile as buffer resources: num_records covers the
// panel's valid rows only, so a load from a row past the operand's end (the
// ragged last row tile, pad columns of the vocabulary) returns zeros.
//
// Load i (0..7) of wave w fills LDS slots q = 64 (8w + i) + l, i.e. row
// r = 64w + 8i + l/8, slot l%8, with chunk (l%8) ^ swz(r) of that row; swz(r)
// depends on i only through its parity, so two base offsets serve all eight.
struct Panels {
  __amdgpu_buffer_rsrc_t a;
  __amdgpu_buffer_rsrc_t b;
  int offa[2];  // byte offsets of this lane's loads 0 and 1 in the A panel
  int offb[2];
  int stepa;    // byte offset between loads i and i+2 (16 rows)
  int stepb;
};

constexpr int kRsrcWord3 = 0x00020000;  // gfx9 raw buffer: 32-bit data format, no swizzle
constexpr int kNoLoad = 0x40000000;     // added to an offset: past every num_records, the load fetches nothing

__device__ __forceinline__ Panels make_panels(const Geo& g, int64_t row0, int64_t col0) {
  Panels p;
  const int64_t ra = g.n_rows - row0;
  const int rows_a = static_cast<int>(ra < BM ? ra : BM);
  p.a = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(g.h + row0 * g.ldh), 0,
                                          static_cast<int>(rows_a * g.ldh * 2), kRsrcWord3);
  const int64_t rb = g.w_end - col0;
  const int rows_b = static_cast<int>(rb <= 0 ? 0 : (rb < BN ? rb : BN));
  const uint16_t* wb = rows_b > 0 ? g.w + (col0 - g.col_base) * g.ldw : g.w;
  p.b = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wb), 0, static_cast<int>(rows_b * g.ldw * 2),
                                          kRsrcWord3);
  const int l = static_cast<int>(threadIdx.x) & 63;
  const int w = static_cast<int>(threadIdx.x) >> 6;
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int r = 64 * w + 8 * par + (l >> 3);
    const int c = (l & 7) ^ swz(r);
    p.offa[par] = r * static_cast<int>(g.ldh) * 2 + c * 16;
    p.offb[par] = r * static_cast<int>(g.ldw) * 2 + c * 16;
  }
  p.stepa = 16 * static_cast<int>(g.ldh) * 2;
  p.stepb = 16 * static_cast<int>(g.ldw) * 2;
  return p;
}

typedef __attribute__((address_space(3))) void* LdsPtr;

// The 8 loads of one operand's BM x 64 stage at byte offset koff (K offset
// times 2, or kNoLoad) into the LDS stage s.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6); }

__device__ __forceinline__ void load_one(__amdgpu_buffer_rsrc_t r, const int (&off)[2], int step, int koff,
                                         uint16_t* __restrict__ s, int i) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)(s + (8 * wave_id() + i) * 512), 16,
                                           off[i & 1] + (i >> 1) * step + koff, 0, 0, 0);
}

__device__ __forceinline__ void load_panel(__amdgpu_buffer_rsrc_t r, const int (&off)[2], int step, int koff,
                                           uint16_t* __restrict__ s) {
#pragma unroll
  for (int i = 0; i < kChunks; ++i) load_one(r, off, step, koff, s, i);
}

// Waits for this wave's LDS operations and panel loads, then for the whole
// workgroup. The memory clobber keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Fragments of K step kk (16 deep) of a stage: for the 32-row block i, lane
// l holds row 32i + l%32, k = 16 kk + 8 (l/32) .. +7, i.e. chunk 2kk + l/32
// (the same shape for the vocabulary rows of the B operand).
__device__ __forceinline__ void load_frags(const uint16_t* __restrict__ sa, const uint16_t* __restrict__ sb, int wm,
                                           int wn, int kk, bf16x8 (&a)[kMB], bf16x8 (&b)[kNB]) {
  const int lane = threadIdx.x & 63;
  const int fr = lane & 31;
  const int slot = ((2 * kk + (lane >> 5)) ^ swz(fr)) * 8;
#pragma unroll
  for (int i = 0; i < kMB; ++i)
    a[i] = *reinterpret_cast<const bf16x8*>(sa + (wm * kWaveM + i * 32 + fr) * kLdsRow + slot);
#pragma unroll
  for (int j = 0; j < kNB; ++j)
    b[j] = *reinterpret_cast<const bf16x8*>(sb + (wn * kWaveN + j * 32 + fr) * kLdsRow + slot);
}

// One K step by hand: MFMA slot t (block t/4, t%4) is followed by the read
// of next-step fragment t (t < 8: A blocks 0-3, then B blocks 0-3) and, when
// the step carries the panel loads, by load t of the next panels (t < 8: the
// hidden-state panel, then the vocabulary panel). sched_barrier keeps the
// compiler from regrouping them.
template <bool kPanel>
__device__ __forceinline__ void mma_step(const bf16x8 (&a)[kMB], const bf16x8 (&b)[kNB], Acc (&acc)[kMB][kNB],
                                         const uint16_t* __restrict__ na_src, const uint16_t* __restrict__ nb_src,
                                         int wm, int wn, int kk, bf16x8 (&na)[kMB], bf16x8 (&nb)[kNB],
                                         const Panels& p, int koff, uint16_t* __restrict__ la,
                                         uint16_t* __restrict__ lb) {
  const int lane = threadIdx.x & 63;
  const int fr = lane & 31;
  const int slot = ((2 * kk + (lane >> 5)) ^ swz(fr)) * 8;
#pragma unroll
  for (int t = 0; t < kMB * kNB; ++t) {
    const int i = t / kNB;
    const int j = t % kNB;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    if (t < kMB)
      na[t] = *reinterpret_cast<const bf16x8*>(na_src + (wm * kWaveM + t * 32 + fr) * kLdsRow + slot);
    else if (t < kMB + kNB)
      nb[t - kMB] = *reinterpret_cast<const bf16x8*>(nb_src + (wn * kWaveN + (t - kMB) * 32 + fr) * kLdsRow + slot);
    if (kPanel) {
      if (t < 8)
        load_one(p.a, p.offa, p.stepa, koff, la, t);
      else
        load_one(p.b, p.offb, p.stepb, koff, lb, t - 8);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Logits of one tile, rounded to BF16, into sO [BM][kOutRow]. Accumulator
// element 4q + e of block (i, j) is row 32i + 8q + 4(l/32) + e, column
// 32j + l%32 of the wave's part.
//
// Stage kt multiplies from LDS buffer kt&1 in 4 steps; the fragments of step
// s+1 (of step 0 of stage kt+1 during step 3) are read during step s. The
// barrier before step 3 waits for the loads of stage kt+1 (issued in step 3
// of stage kt-1) and for every wave's reads of buffer kt&1; step 3 then loads
// stage kt+2 into that buffer. Past the last stage the loads fetch nothing.
__device__ __forceinline__ void tile_logits(const Geo& g, int64_t row0, int64_t col0, uint16_t* __restrict__ smem,
                                            uint16_t* __restrict__ sO) {
  uint16_t* sa = smem;                  // [2][kStage]
  uint16_t* sb = smem + 2 * kStage;     // [2][kStage]
  const int wave = threadIdx.x >> 6;
  const int wm = wave % (BM / kWaveM);
  const int wn = wave / (BM / kWaveM);
  Acc acc[kMB][kNB];
#pragma unroll
  for (int i = 0; i < kMB; ++i)
#pragma unroll
    for (int j = 0; j < kNB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  const Panels p = make_panels(g, row0, col0);
  const int kt_n = g.d / BK;
  load_panel(p.a, p.offa, p.stepa, 0, sa);
  load_panel(p.b, p.offb, p.stepb, 0, sb);
  const int k1 = kt_n > 1 ? BK * 2 : kNoLoad;
  load_panel(p.a, p.offa, p.stepa, k1, sa + kStage);
  load_panel(p.b, p.offb, p.stepb, k1, sb + kStage);
  asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");  // stage 0 landed
  bf16x8 fa[2][kMB], fb[2][kNB];
  load_frags(sa, sb, wm, wn, 0, fa[0], fb[0]);
  for (int kt = 0; kt < kt_n; ++kt) {
    const int cur = kt & 1;
    uint16_t* ca = sa + cur * kStage;
    uint16_t* cb = sb + cur * kStage;
    mma_step<false>(fa[0], fb[0], acc, ca, cb, wm, wn, 1, fa[1], fb[1], p, 0, ca, cb);
    mma_step<false>(fa[1], fb[1], acc, ca, cb, wm, wn, 2, fa[0], fb[0], p, 0, ca, cb);
    mma_step<false>(fa[0], fb[0], acc, ca, cb, wm, wn, 3, fa[1], fb[1], p, 0, ca, cb);
    stage_barrier();
    const int k2 = kt + 2 < kt_n ? (kt + 2) * BK * 2 : kNoLoad;
    mma_step<true>(fa[1], fb[1], acc, sa + (cur ^ 1) * kStage, sb + (cur ^ 1) * kStage, wm, wn, 0, fa[0], fb[0], p,
                   k2, ca, cb);
  }
  stage_barrier();  // the epilogue tile overwrites the stages (the loads past the end write zeros)

  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kMB; ++i)
#pragma unroll
    for (int j = 0; j < kNB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = wm * kWaveM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int c = wn * kWaveN + j * 32 + (lane & 31);
        const __bf16 v = static_cast<__bf16>(acc[i][j][e]);
        sO[r * kOutRow + c] = __builtin_bit_cast(uint16_t, v);
      }
  __syncthreads();
}

// Summary of columns [q*SN, (q+1)*SN) of row r of the tile; two neighbouring
// threads share an item, 64 columns each.
__device__ __forceinline__ void row_summary(const Geo& g, int64_t row0, int64_t tcol0, int r, int q,
                                            const uint16_t* __restrict__ sO, const float* __restrict__ temperature,
                                            const int64_t* __restrict__ target, ShardSummary* __restrict__ ws) {
  const int half = threadIdx.x & 1;
  const int64_t col0 = tcol0 + q * SN;
  const int64_t n_t = (col0 - g.col_base) / SN;  // summary index in this launch
  const int64_t gr = row0 + r;
  const bool row_ok = gr < g.n_rows;
  const float t = row_ok ? temperature[gr] : 1.0f;
  const int64_t tg = row_ok ? target[gr] : -1;
  const int64_t cb = col0 + half * 64;
  int64_t nv64 = g.w_end - cb;
  const int nvalid = static_cast<int>(nv64 < 0 ? 0 : (nv64 > 64 ? 64 : nv64));
  const uint16_t* src = sO + r * kOutRow + q * SN + half * 64;
  // pass 1: maximum (and, for greedy rows, NaN/+inf and the first maximum)
  float m = -INFINITY;
  bool bad = false;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(src + v * 8);
    float x[8];
    rlk::unpack8(q, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool ok = v * 8 + e < nvalid;
      bad |= ok && ((x[e] != x[e]) || (x[e] == INFINITY));
      m = ok ? fmaxf(m, x[e]) : m;
    }
  }
  m = fmaxf(m, __shfl_xor(m, 1));
  bad = bad || (__shfl_xor(static_cast<int>(bad), 1) != 0);
  ShardSummary s;
  s.r = 0.0f;
  s.l = 0.0f;
  s.m = m;
  s.aux = -1;
  if (!rlk::temperature_valid(t)) {
    s.l = NAN;
  } else if (t == 0.0f) {
    int first = INT32_MAX;
    for (int j = 0; j < nvalid; ++j) {
      const float x = __uint_as_float(static_cast<uint32_t>(src[j]) << 16);
      if (x == m) {
        first = static_cast<int>(cb) + j;
        break;
      }
    }
    const int other = __shfl_xor(first, 1);
    first = other < first ? other : first;
    s.l = bad ? NAN : 0.0f;
    s.aux = (first == INT32_MAX) ? -1 : first;
  } else {
    const float c = rlk::kLog2e / t;
    const float rr = rlk::ref_exponent(m, c);
    float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(src + v * 8);
      float x[8];
      rlk::unpack8(q, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float term = __builtin_amdgcn_exp2f(fmaf(x[e], c, -rr));
        a4[e & 3] += (v * 8 + e < nvalid) ? term : 0.0f;
      }
    }
    const float mine = (a4[0] + a4[1]) + (a4[2] + a4[3]);
    const float other = __shfl_xor(mine, 1);
    s.r = rr;
    s.l = half == 0 ? mine + other : other + mine;
    if (tg >= col0 && tg < col0 + SN && tg < g.vocab_real)
      s.aux = static_cast<int32_t>(sO[r * kOutRow + q * SN + static_cast<int>(tg - col0)]);
  }
  if (row_ok && half == 0) ws[gr * g.n_sum + n_t] = s;
}

__device__ __forceinline__ void tile_summaries(const Geo& g, int64_t row0, int64_t col0,
                                               const uint16_t* __restrict__ sO, const float* __restrict__ temperature,
                                               const int64_t* __restrict__ target, ShardSummary* __restrict__ ws) {
  // (BM rows) x (BN / SN summaries) items, two threads each
  for (int item = threadIdx.x >> 1; item < BM * (BN / SN); item += kThreads / 2) {
    const int r = item % BM;
    const int q = item / BM;
    if (col0 + q * SN < g.col_end) row_summary(g, row0, col0, r, q, sO, temperature, target, ws);
  }
}

// Stores the BF16 tile; real columns from the tile, pads -inf.
__device__ __forceinline__ void tile_store(const Geo& g, int64_t row0, int64_t col0, const uint16_t* __restrict__ sO,
                                           uint16_t* __restrict__ out, int64_t ldo) {
  for (int c = threadIdx.x; c < BM * (BN / 8); c += kThreads) {
    const int r = c / (BN / 8);
    const int ch = c % (BN / 8);
    const int64_t gr = row0 + r;
    const int64_t gc = col0 + ch * 8;
    if (gr >= g.n_rows || gc >= g.vocab_padded) continue;
    u32x4 v = *reinterpret_cast<const u32x4*>(sO + r * kOutRow + ch * 8);
    if (gc + 8 > g.vocab_real) {
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t lo = (gc + 2 * h < g.vocab_real) ? (w[h] & 0xFFFFu) : 0xFF80u;
        const uint32_t hi = (gc + 2 * h + 1 < g.vocab_real) ? (w[h] & 0xFFFF0000u) : 0xFF800000u;
        w[h] = lo | hi;
      }
      v = u32x4{w[0], w[1], w[2], w[3]};
    }
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + gr * ldo + gc));
  }
}

__host__ __device__ __forceinline__ int64_t virtual_blocks(const Geo& g) {
  const int64_t groups = g.m_groups * g.n_groups;
  return ((groups + kXcds - 1) / kXcds) * kXcds * kGM * kGN;
}

template <bool kLogp>
__global__ __launch_bounds__(kThreads) void k_linear(Geo g, const float* __restrict__ temperature,
                                                     const int64_t* __restrict__ target,
                                                     ShardSummary* __restrict__ ws, uint16_t* __restrict__ out,
                                                     int64_t ldo) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[kSmem];
  uint16_t* sO = smem;  // the epilogue tile reuses the stages
  const int64_t n_virtual = virtual_blocks(g);
  for (int64_t v = blockIdx.x; v < n_virtual; v += gridDim.x) {  // uniform across the workgroup
    int64_t m_t, n_t;
    if (!tile_of(g, v, m_t, n_t)) continue;
    const int64_t row0 = m_t * BM;
    const int64_t col0 = g.col_base + n_t * BN;
    tile_logits(g, row0, col0, smem, sO);
    if (kLogp)
      tile_summaries(g, row0, col0, sO, temperature, target, ws);
    else
      tile_store(g, row0, col0, sO, out, ldo);
    __syncthreads();  // sO is overwritten by the next tile's first stage
  }
}

// Summary k (global column order) of a row in rank-major storage: rank
// k / per_rank holds n_rows x per_rank records.
__device__ __forceinline__ const ShardSummary& summary_at(const ShardSummary* __restrict__ ws, int64_t n_rows,
                                                          int64_t per_rank, int64_t row, int64_t k) {
  return ws[((k / per_rank) * n_rows + row) * per_rank + k % per_rank];
}

// One wave per row: the row's 128-column summaries merged in column order.
__global__ __launch_bounds__(256) void k_lin_merge(const ShardSummary* __restrict__ ws, int64_t n_rows,
                                                   int64_t n_sum, int64_t per_rank, int64_t vocab_real,
                                                   const float* __restrict__ temperature,
                                                   const int64_t* __restrict__ target, float* __restrict__ logp_out,
                                                   float* __restrict__ lse_out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;  // uniform across the wave
  const float t = temperature[row];
  const int64_t tg = target[row];
  float logp = NAN;
  float lse = NAN;
  if (rlk::temperature_valid(t) && tg >= 0 && tg < vocab_real) {
    if (t == 0.0f) {
      float m = -INFINITY;
      bool bad = false;
      for (int64_t k = lane; k < n_sum; k += 64) {
        const ShardSummary sk = summary_at(ws, n_rows, per_rank, row, k);
        m = fmaxf(m, sk.m);
        bad |= (sk.l != sk.l);
      }
      m = rlk::wave_max(m);
      bad = __any(bad);
      int64_t first = INT64_MAX;
      for (int64_t k = lane; k < n_sum; k += 64)
        if (summary_at(ws, n_rows, per_rank, row, k).m == m) {
          first = k;
          break;
        }
      for (int o = 32; o >= 1; o >>= 1) {
        const int64_t other = __shfl_xor(first, o);
        first = other < first ? other : first;
      }
      if (!bad && m != -INFINITY && first != INT64_MAX)
        logp = (static_cast<int64_t>(summary_at(ws, n_rows, per_rank, row, first).aux) == tg) ? 0.0f : -INFINITY;
    } else {
      float rmax = -INFINITY;
      for (int64_t k = lane; k < n_sum; k += 64) {
        const ShardSummary sk = summary_at(ws, n_rows, per_rank, row, k);
        if (sk.l > 0.0f || sk.l != sk.l) rmax = fmaxf(rmax, sk.r);
      }
      rmax = rlk::wave_max(rmax);
      double acc = 0.0;
      bool nan = false;
      for (int64_t k = lane; k < n_sum; k += 64) {
        const ShardSummary sk = summary_at(ws, n_rows, per_rank, row, k);
        if (sk.l == 0.0f) continue;
        const float d = fmaxf(sk.r - rmax, -2000.0f);
        acc = acc + ldexp(static_cast<double>(sk.l), static_cast<int>(d));
        nan |= (sk.r != sk.r) || (sk.l != sk.l);
      }
      for (int o = 32; o >= 1; o >>= 1) acc = acc + __shfl_xor(acc, o);
      nan = __any(nan);
      const int tbits = summary_at(ws, n_rows, per_rank, row, tg / SN).aux;
      if (!nan && acc > 0.0 && acc < INFINITY && rmax > -INFINITY && rmax < INFINITY && tbits >= 0) {
        const double lse2 = static_cast<double>(rmax) + log2(acc);
        const double lse_d = lse2 * rlk::kLn2;
        const float xt = __uint_as_float(static_cast<uint32_t>(tbits) << 16);
        const float zt = xt / t;  // IEEE float32 division, rounded to nearest
        lse = static_cast<float>(lse_d);
        logp = static_cast<float>(static_cast<double>(zt) - lse_d);
      }
    }
  }
  if (lane == 0) {
    logp_out[row] = logp;
    if (lse_out) lse_out[row] = lse;
  }
}

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static int32_t launched() { return hipGetLastError() == hipSuccess ? RLK_OK : RLK_ERR_HIP; }

static int32_t check_layout(int64_t n_rows, const rlk_vocab_layout* L) {
  if (L == nullptr) return RLK_ERR_NULL;
  if (n_rows < 0 || n_rows > kMaxRows) return RLK_ERR_SHAPE;
  if (L->n_shards != 8) return RLK_ERR_SHAPE;
  if (L->vocab_padded < 64 || L->vocab_padded > kMaxVocab || L->vocab_padded % 64 != 0) return RLK_ERR_SHAPE;
  if (L->vocab_real < 1 || L->vocab_real > L->vocab_padded) return RLK_ERR_SHAPE;
  if (L->row_stride < L->vocab_padded || L->row_stride % 8 != 0) return RLK_ERR_SHAPE;
  if (!(L->groups == 1 || L->groups == 2 || L->groups == 4 || L->groups == 8)) return RLK_ERR_GROUPS;
  return RLK_OK;
}

static int32_t check_operands(int64_t n_rows, int64_t d, int64_t ldh, int64_t ldw, const rlk_vocab_layout* L) {
  if (d < 64 || d > kMaxD || d % BK != 0) return RLK_ERR_SHAPE;
  if (ldh < d || ldh % 8 != 0 || ldw < d || ldw % 8 != 0) return RLK_ERR_SHAPE;
  if (ldh > kMaxLd || ldw > kMaxLd) return RLK_ERR_SHAPE;
  if (n_rows > 0 && ldh > INT64_MAX / 2 / n_rows) return RLK_ERR_SHAPE;
  if (ldw > INT64_MAX / 2 / L->vocab_real) return RLK_ERR_SHAPE;
  return RLK_OK;
}

static Geo make_geo(const uint16_t* h, int64_t n_rows, int64_t d, int64_t ldh, const uint16_t* w, int64_t ldw,
                    const rlk_vocab_layout* L, int64_t col_base, int64_t col_end) {
  Geo g;
  g.h = h;
  g.w = w;
  g.ldh = ldh;
  g.ldw = ldw;
  g.n_rows = n_rows;
  g.vocab_real = L->vocab_real;
  g.vocab_padded = L->vocab_padded;
  g.d = static_cast<int>(d);
  g.m_tiles = static_cast<int>((n_rows + BM - 1) / BM);
  g.col_base = col_base;
  g.col_end = col_end;
  g.w_end = col_end < L->vocab_real ? col_end : L->vocab_real;
  g.n_tiles = (col_end - col_base + BN - 1) / BN;
  g.n_sum = (col_end - col_base + SN - 1) / SN;
  g.m_groups = (g.m_tiles + kGM - 1) / kGM;
  g.n_groups = (g.n_tiles + kGN - 1) / kGN;
  return g;
}

static unsigned grid_for(const Geo& g) {
  const int64_t v = virtual_blocks(g);
  return static_cast<unsigned>(v < kMaxGrid ? v : kMaxGrid);
}

}  // namespace rlk_lin

extern "C" {

size_t rlk_linear_logp_workspace_bytes(int64_t n_rows, const rlk_vocab_layout* layout) {
  using namespace rlk_lin;
  if (check_layout(n_rows, layout) != RLK_OK) return 0;
  return static_cast<size_t>(n_rows) * static_cast<size_t>((layout->vocab_padded + SN - 1) / SN) *
         sizeof(ShardSummary);
}

int32_t rlk_linear(const uint16_t* hidden, int64_t n_rows, int64_t d_model, int64_t hidden_stride,
                   const uint16_t* weight, int64_t weight_stride, const rlk_vocab_layout* layout,
                   uint16_t* logits_out, hipStream_t stream) {
  using namespace rlk_lin;
  int32_t st = check_layout(n_rows, layout);
  if (st != RLK_OK) return st;
  if ((st = check_operands(n_rows, d_model, hidden_stride, weight_stride, layout)) != RLK_OK) return st;
  if (n_rows > 0 && layout->row_stride > INT64_MAX / 2 / n_rows) return RLK_ERR_SHAPE;
  if (n_rows == 0) return RLK_OK;
  if (!hidden || !weight || !logits_out) return RLK_ERR_NULL;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(logits_out, 16)) return RLK_ERR_ALIGN;
  const Geo g = make_geo(hidden, n_rows, d_model, hidden_stride, weight, weight_stride, layout, 0,
                         layout->vocab_padded);
  k_linear<false><<<dim3(grid_for(g)), dim3(kThreads), 0, stream>>>(g, nullptr, nullptr, nullptr, logits_out,
                                                                     layout->row_stride);
  return launched();
}

int32_t rlk_linear_logp(const uint16_t* hidden, int64_t n_rows, int64_t d_model, int64_t hidden_stride,
                        const uint16_t* weight, int64_t weight_stride, const rlk_vocab_layout* layout,
                        const float* temperature, const int64_t* target, float* logp_out, float* lse_out,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace rlk_lin;
  int32_t st = check_layout(n_rows, layout);
  if (st != RLK_OK) return st;
  if ((st = check_operands(n_rows, d_model, hidden_stride, weight_stride, layout)) != RLK_OK) return st;
  if (n_rows == 0) return RLK_OK;
  if (!hidden || !weight || !temperature || !target || !logp_out || !workspace) return RLK_ERR_NULL;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(workspace, 16) || !aligned(temperature, 4) ||
      !aligned(target, 8) || !aligned(logp_out, 4) || (lse_out && !aligned(lse_out, 4)))
    return RLK_ERR_ALIGN;
  if (workspace_bytes < rlk_linear_logp_workspace_bytes(n_rows, layout)) return RLK_ERR_WORKSPACE;
  const Geo g = make_geo(hidden, n_rows, d_model, hidden_stride, weight, weight_stride, layout, 0,
                         layout->vocab_padded);
  ShardSummary* ws = static_cast<ShardSummary*>(workspace);
  k_linear<true><<<dim3(grid_for(g)), dim3(kThreads), 0, stream>>>(g, temperature, target, ws, nullptr, 0);
  if ((st = launched()) != RLK_OK) return st;
  k_lin_merge<<<dim3(static_cast<unsigned>((n_rows + 3) / 4)), dim3(256), 0, stream>>>(
      ws, n_rows, g.n_sum, g.n_sum, layout->vocab_real, temperature, target, logp_out, lse_out);
  return launched();
}

size_t rlk_linear_logp_summary_bytes(int64_t n_rows, const rlk_vocab_layout* layout) {
  using namespace rlk_lin;
  if (check_layout(n_rows, layout) != RLK_OK) return 0;
  const int64_t cols = layout->vocab_padded / layout->groups;
  if (cols % SN != 0) return 0;
  return static_cast<size_t>(n_rows) * static_cast<size_t>(cols / SN) * sizeof(ShardSummary);
}

int32_t rlk_linear_logp_summaries(const uint16_t* hidden, int64_t n_rows, int64_t d_model, int64_t hidden_stride,
                                  const uint16_t* weight_shard, int64_t weight_stride, const rlk_vocab_layout* layout,
                                  int32_t rank, const float* temperature, const int64_t* target,
                                  void* summaries_out, size_t summaries_bytes, hipStream_t stream) {
  using namespace rlk_lin;
  int32_t st = check_layout(n_rows, layout);
  if (st != RLK_OK) return st;
  if ((st = check_operands(n_rows, d_model, hidden_stride, weight_stride, layout)) != RLK_OK) return st;
  const int64_t cols = layout->vocab_padded / layout->groups;
  if (cols % SN != 0 || rank < 0 || rank >= layout->groups) return RLK_ERR_SHAPE;
  if (n_rows == 0) return RLK_OK;
  if (!hidden || !weight_shard || !temperature || !target || !summaries_out) return RLK_ERR_NULL;
  if (!aligned(hidden, 16) || !aligned(weight_shard, 16) || !aligned(summaries_out, 16) ||
      !aligned(temperature, 4) || !aligned(target, 8))
    return RLK_ERR_ALIGN;
  if (summaries_bytes < rlk_linear_logp_summary_bytes(n_rows, layout)) return RLK_ERR_WORKSPACE;
  const int64_t col_base = static_cast<int64_t>(rank) * cols;
  const Geo g = make_geo(hidden, n_rows, d_model, hidden_stride, weight_shard, weight_stride, layout, col_base,
                         col_base + cols);
  k_linear<true><<<dim3(grid_for(g)), dim3(kThreads), 0, stream>>>(g, temperature, target,
                                                                    static_cast<ShardSummary*>(summaries_out),
                                                                    nullptr, 0);
  return launched();
}

int32_t rlk_linear_logp_merge(const void* summaries, size_t summaries_bytes, int64_t n_rows,
                              const rlk_vocab_layout* layout, const float* temperature, const int64_t* target,
                              float* logp_out, float* lse_out, hipStream_t stream) {
  using namespace rlk_lin;
  int32_t st = check_layout(n_rows, layout);
  if (st != RLK_OK) return st;
  const int64_t cols = layout->vocab_padded / layout->groups;
  if (cols % SN != 0) return RLK_ERR_SHAPE;
  if (n_rows == 0) return RLK_OK;
  if (!summaries || !temperature || !target || !logp_out) return RLK_ERR_NULL;
  if (!aligned(summaries, 16) || !aligned(temperature, 4) || !aligned(target, 8) || !aligned(logp_out, 4) ||
      (lse_out && !aligned(lse_out, 4)))
    return RLK_ERR_ALIGN;
  if (summaries_bytes < rlk_linear_logp_summary_bytes(n_rows, layout) * static_cast<size_t>(layout->groups))
    return RLK_ERR_WORKSPACE;
  k_lin_merge<<<dim3(static_cast<unsigned>((n_rows + 3) / 4)), dim3(256), 0, stream>>>(
      static_cast<const ShardSummary*>(summaries), n_rows, layout->vocab_padded / SN, cols / SN,
      layout->vocab_real, temperature, target, logp_out, lse_out);
  return launched();
}

}  // extern "C"
