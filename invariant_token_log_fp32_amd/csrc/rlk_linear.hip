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
//   k_linear<kLogp>  one 256 x 256 tile of logits per step of a loop over
//                    tiles (one workgroup per compute unit), in XCD-aware
//                    groups of 4 x 8 tiles
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
//                    reads). Fragments are read two steps ahead (four sets in
//                    registers), so a stage's buffer is free after step 1:
//                    one barrier per stage, there, after the next stage's
//                    loads have landed; steps 2 and 3 then load the stage
//                    after next into the freed buffer, which spreads the LDS
//                    writes over half of the stage.
//                    The MFMA takes the vocabulary fragment first, so a lane
//                    holds 4 consecutive columns of one row per accumulator
//                    quad and a row's 128 columns of a wave sit in two lanes.
//                    Epilogue, from the registers (no LDS, so the next
//                    tile's first two stages load meanwhile): the fp32
//                    accumulators rounded to BF16 and either stored
//                    (rlk_linear) or reduced per row to a 16-byte summary of
//                    the wave's 128 columns (rlk_linear_logp): integer
//                    reference exponent r from their exact maximum and l =
//                    sum of 2^(x*c - r) in a fixed order; greedy rows keep
//                    the maximum and its lowest column.
//   k_lin_merge      one wave per row: the row's 128-column summaries merged
//                    in column order (fp64), then the target's logprob.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

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
constexpr int kSmem = 4 * kStage;       // bf16: two stages of both operands
static_assert(SN == kWaveN, "one summary per row of a wave's part");
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
  // The offsets do not depend on the tile; without this the compiler hoists
  // the 32 per-load offsets out of the loop over tiles, spills them, and each
  // reload then waits behind the panel loads already in flight.
  asm volatile("" : "+v"(p.offa[0]), "+v"(p.offa[1]), "+v"(p.offb[0]), "+v"(p.offb[1]));
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
// of fragment t of the step after next (t < 8: A blocks 0-3, then B blocks
// 0-3) and, after every other slot, when the step carries panel loads, by one
// load of the next panels (kPanel 1: the hidden-state panel's 8, 2: the
// vocabulary panel's). sched_barrier keeps the compiler from regrouping them.
template <int kPanel>
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
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    if (t < kMB)
      na[t] = *reinterpret_cast<const bf16x8*>(na_src + (wm * kWaveM + t * 32 + fr) * kLdsRow + slot);
    else if (t < kMB + kNB)
      nb[t - kMB] = *reinterpret_cast<const bf16x8*>(nb_src + (wn * kWaveN + (t - kMB) * 32 + fr) * kLdsRow + slot);
    if (kPanel && (t & 1) == 0) {
      if (kPanel == 1)
        load_one(p.a, p.offa, p.stepa, koff, la, t >> 1);
      else
        load_one(p.b, p.offb, p.stepb, koff, lb, t >> 1);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Panels of stages 0 and 1 of a tile into LDS buffers par and par ^ 1
// (stage 1 only when the tile has it).
__device__ __forceinline__ void prefetch_tile(const Panels& p, int kt_n, int par, uint16_t* __restrict__ smem) {
  load_panel(p.a, p.offa, p.stepa, 0, smem + par * kStage);
  load_panel(p.b, p.offb, p.stepb, 0, smem + (2 + par) * kStage);
  const int k1 = kt_n > 1 ? BK * 2 : kNoLoad;
  load_panel(p.a, p.offa, p.stepa, k1, smem + (par ^ 1) * kStage);
  load_panel(p.b, p.offb, p.stepb, k1, smem + (2 + (par ^ 1)) * kStage);
}

// Logits of one tile (fp32) into acc. The tile's stage kt lives in LDS
// buffer (kt + par) & 1; on entry stages 0 and 1 are loaded or in flight and
// the fragments of steps 0 and 1 of stage 0 are in fa[0..1], fb[0..1]. The
// MFMA takes the vocabulary fragment as its first operand, so block (i, j)
// holds the transposed product: element 4q + e of lane l is row 32i + l%32,
// column 32j + 8q + 4(l/32) + e of the wave's part.
//
// Stage kt multiplies in 4 steps; the fragments of step s+2 (of steps 0 and
// 1 of the next stage during steps 2 and 3) are read during step s. The
// barrier after step 1 waits for the loads of the next stage (issued in steps
// 2 and 3 of the stage before) and for every wave's reads of this stage's
// buffer; steps 2 and 3 then load, into that buffer, the stage two ahead:
// stage kt+2 of this tile, or, in the last two stages, stage 0 or 1 of the
// next tile (pn) when there is one and the tile has two stages or more, else
// nothing. So on return the next tile's stages 0 and 1 are loaded or in
// flight and its first fragments are in fa, fb, with no pause between tiles.
__device__ __forceinline__ void tile_logits(const Geo& g, const Panels& p, const Panels& pn, bool next, int par,
                                            uint16_t* __restrict__ smem, Acc (&acc)[kMB][kNB],
                                            bf16x8 (&fa)[kSteps][kMB], bf16x8 (&fb)[kSteps][kNB]) {
  uint16_t* sa = smem;                  // [2][kStage]
  uint16_t* sb = smem + 2 * kStage;     // [2][kStage]
  const int wave = threadIdx.x >> 6;
  const int wm = wave % (BM / kWaveM);
  const int wn = wave / (BM / kWaveM);
#pragma unroll
  for (int i = 0; i < kMB; ++i)
#pragma unroll
    for (int j = 0; j < kNB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  const int kt_n = g.d / BK;
  const bool ahead = next && kt_n >= 2;
  for (int kt = 0; kt < kt_n; ++kt) {
    const int cur = (kt + par) & 1;
    uint16_t* ca = sa + cur * kStage;
    uint16_t* cb = sb + cur * kStage;
    uint16_t* na = sa + (cur ^ 1) * kStage;
    uint16_t* nb = sb + (cur ^ 1) * kStage;
    mma_step<0>(fa[0], fb[0], acc, ca, cb, wm, wn, 2, fa[2], fb[2], p, 0, ca, cb);
    mma_step<0>(fa[1], fb[1], acc, ca, cb, wm, wn, 3, fa[3], fb[3], p, 0, ca, cb);
    stage_barrier();
    const bool own = kt + 2 < kt_n;
    Panels q = p;
    q.a = own ? p.a : pn.a;
    q.b = own ? p.b : pn.b;
    const int k2 = own ? (kt + 2) * BK * 2 : (ahead ? (kt + 2 - kt_n) * BK * 2 : kNoLoad);
    mma_step<1>(fa[2], fb[2], acc, na, nb, wm, wn, 0, fa[0], fb[0], q, k2, ca, cb);
    mma_step<2>(fa[3], fb[3], acc, na, nb, wm, wn, 1, fa[1], fb[1], q, k2, ca, cb);
  }
}

// BF16 bits of an fp32 value, rounded to nearest even, as a float.
__device__ __forceinline__ float round_bf16(float v) {
  const __bf16 b = static_cast<__bf16>(v);
  return __uint_as_float(static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to BF16 (nearest even) in one 32-bit word, low first.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// 8 BF16 logits (4 packed pairs) at column c of a row; pad columns -inf.
__device__ __forceinline__ void store8(const Geo& g, uint16_t* __restrict__ dst, int64_t c, uint32_t w0, uint32_t w1,
                                      uint32_t w2, uint32_t w3) {
  if (c + 8 > g.vocab_real) {
    const uint32_t w[4] = {w0, w1, w2, w3};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = (c + 2 * k < g.vocab_real) ? (w[k] & 0xFFFFu) : 0xFF80u;
      const uint32_t hi = (c + 2 * k + 1 < g.vocab_real) ? (w[k] & 0xFFFF0000u) : 0xFF800000u;
      o[k] = lo | hi;
    }
    w0 = o[0];
    w1 = o[1];
    w2 = o[2];
    w3 = o[3];
  }
  *reinterpret_cast<u32x4*>(dst) = u32x4{w0, w1, w2, w3};
}

// The 16 BF16 logits of block (i, j) that lane l stores, as 8 packed words:
// lane l holds, for q = 0..3, columns 8q + 4h .. +3 (h = l/32) of row l%32;
// one exchange with lane l^32 gives it the 16 columns 16h .. +15.
__device__ __forceinline__ void block_words(const Acc& v, int h, uint32_t (&w)[8]) {
  // columns 8q + 4h + (0, 1) and (2, 3) of this lane, q = 0..3
  const uint32_t p00 = pack_bf16(v[0], v[1]), p01 = pack_bf16(v[2], v[3]);
  const uint32_t p10 = pack_bf16(v[4], v[5]), p11 = pack_bf16(v[6], v[7]);
  const uint32_t p20 = pack_bf16(v[8], v[9]), p21 = pack_bf16(v[10], v[11]);
  const uint32_t p30 = pack_bf16(v[12], v[13]), p31 = pack_bf16(v[14], v[15]);
  // h = 0 keeps q = 0, 1 and takes the partner's; h = 1 keeps q = 2, 3
  const uint32_t g00 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(h ? p00 : p20), 32));
  const uint32_t g01 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(h ? p01 : p21), 32));
  const uint32_t g10 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(h ? p10 : p30), 32));
  const uint32_t g11 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(h ? p11 : p31), 32));
  const uint32_t a0 = h ? p20 : p00, a1 = h ? p21 : p01;
  const uint32_t b0 = h ? p30 : p10, b1 = h ? p31 : p11;
  w[0] = h ? g00 : a0;
  w[1] = h ? g01 : a1;
  w[2] = h ? a0 : g00;
  w[3] = h ? a1 : g01;
  w[4] = h ? g10 : b0;
  w[5] = h ? g11 : b1;
  w[6] = h ? b0 : g10;
  w[7] = h ? b1 : g11;
}

// Stores the tile's BF16 logits from the accumulators; pads -inf.
__device__ __forceinline__ void tile_store(const Geo& g, int64_t row0, int64_t col0, const Acc (&acc)[kMB][kNB],
                                           uint16_t* __restrict__ out, int64_t ldo) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const int wm = wave % (BM / kWaveM);
  const int wn = wave / (BM / kWaveM);
  const int64_t cw = col0 + wn * kWaveN + 16 * h;  // this lane's first column of block j = 0
  if (col0 + BN <= g.vocab_real) {                 // uniform: every column of the tile is real
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
      const int64_t gr = row0 + wm * kWaveM + i * 32 + (lane & 31);
      u32x4* dst = reinterpret_cast<u32x4*>(out + gr * ldo + cw);
#pragma unroll
      for (int j = 0; j < kNB; ++j) {
        uint32_t w[8];
        block_words(acc[i][j], h, w);
        // ordinary stores: L2 merges the 16-byte pieces of a row into whole lines
        // (with the non-temporal hint they reach HBM as partial lines, 15% slower)
        if (gr < g.n_rows) {
          dst[4 * j] = u32x4{w[0], w[1], w[2], w[3]};
          dst[4 * j + 1] = u32x4{w[4], w[5], w[6], w[7]};
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < kMB; ++i) {
    const int64_t gr = row0 + wm * kWaveM + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      uint32_t w[8];
      block_words(acc[i][j], h, w);
      const int64_t gc = cw + j * 32;
      if (gr >= g.n_rows || gc >= g.vocab_padded) continue;
      store8(g, out + gr * ldo + gc, gc, w[0], w[1], w[2], w[3]);
      store8(g, out + gr * ldo + gc + 8, gc + 8, w[4], w[5], w[6], w[7]);
    }
  }
}

// Per-row summaries of the wave's 128 columns from the accumulators: lane l
// holds 64 of a row's columns (32j + 8q + 4h + e, h = l/32), lane l^32 the
// other 64. Each lane reduces its columns in the order (j, q, e) (the sum in
// four partial sums, k mod 4), then the two halves combine, the h = 0 half
// first. Integer reference exponent r from the exact row maximum; greedy rows
// keep the maximum and its lowest column; the target's BF16 bits when the
// target is one of the columns. The rare cases (a target among the columns,
// a greedy row) run behind branches that are uniform across the wave, so the
// common path stays short.
__device__ __forceinline__ void tile_summaries(const Geo& g, int64_t row0, int64_t col0, const Acc (&acc)[kMB][kNB],
                                               const float (&tr)[kMB], const int64_t (&tgr)[kMB],
                                               ShardSummary* __restrict__ ws) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const int wm = wave % (BM / kWaveM);
  const int wn = wave / (BM / kWaveM);
  const int64_t cb = col0 + wn * kWaveN;  // first column of the summary
  if (cb >= g.col_end) return;            // uniform across the wave
  const int64_t n_t = (cb - g.col_base) / SN;
  int64_t lim64 = g.w_end - cb - 4 * h;   // this lane's column 32j + 8q + e is real iff below lim
  const int lim = static_cast<int>(lim64 < 0 ? 0 : (lim64 > 128 ? 128 : lim64));
  const bool all_real = cb + kWaveN <= g.w_end;  // uniform across the wave
#pragma unroll
  for (int i = 0; i < kMB; ++i) {
    const int64_t gr = row0 + wm * kWaveM + i * 32 + (lane & 31);
    const float t = tr[i];
    const int64_t tg = tgr[i];
    float x[64];
#pragma unroll
    for (int k = 0; k < 64; ++k) x[k] = round_bf16(acc[i][k >> 4][k & 15]);
    if (!all_real) {
      // columns past the real vocabulary: -inf (they follow every real column of the lane)
#pragma unroll
      for (int k = 0; k < 64; ++k) x[k] = (32 * (k >> 4) + 8 * ((k >> 2) & 3) + (k & 3) < lim) ? x[k] : -INFINITY;
    }
    float mx[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) mx[u] = fmaxf(fmaxf(x[4 * u], x[4 * u + 1]), fmaxf(x[4 * u + 2], x[4 * u + 3]));
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int u = 0; u < w; ++u) mx[u] = fmaxf(mx[u], mx[u + w]);
    const float m = fmaxf(mx[0], __shfl_xor(mx[0], 32));
    ShardSummary s;
    s.m = m;
    s.aux = -1;
    // positive temperature
    const float c = rlk::kLog2e / t;
    const float rr = rlk::ref_exponent(m, c);
    float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < 64; ++k) a4[k & 3] += __builtin_amdgcn_exp2f(fmaf(x[k], c, -rr));
    const float mine = (a4[0] + a4[1]) + (a4[2] + a4[3]);
    const float other = __shfl_xor(mine, 32);
    s.r = rr;
    s.l = h == 0 ? mine + other : other + mine;
    const int64_t lc = tg - cb;
    const bool tin = (lc >= 0) && (lc < SN) && (tg < g.vocab_real);
    if (__any(tin)) {
      const int lci = static_cast<int>(tin ? lc : 0);
      const int kt = (tin && ((lci >> 2) & 1) == h) ? (lci >> 5) * 16 + ((lci >> 3) & 3) * 4 + (lci & 3) : -1;
      int tbits = -1;
#pragma unroll
      for (int k = 0; k < 64; ++k) tbits = (k == kt) ? static_cast<int>(__float_as_uint(x[k]) >> 16) : tbits;
      const int otb = __shfl_xor(tbits, 32);
      s.aux = tin ? (tbits >= 0 ? tbits : otb) : -1;
    }
    const bool greedy = (t == 0.0f);
    if (__any(greedy)) {
      // first column holding the maximum, and NaN or +inf among the real columns
      // bitwise operators, not && and ||: no branch per column
      int bad = 0;
      int first = INT32_MAX;
#pragma unroll
      for (int k = 63; k >= 0; --k) {
        const int cl = 32 * (k >> 4) + 8 * ((k >> 2) & 3) + (k & 3);
        const int ok = cl < lim;
        bad |= ok & (static_cast<int>(x[k] != x[k]) | static_cast<int>(x[k] == INFINITY));
        first = (ok & static_cast<int>(x[k] == m)) ? static_cast<int>(cb) + cl + 4 * h : first;
      }
      bad |= __shfl_xor(bad, 32);
      const int ofirst = __shfl_xor(first, 32);
      first = ofirst < first ? ofirst : first;
      if (greedy) {
        s.r = 0.0f;
        s.l = bad ? NAN : 0.0f;
        s.aux = (first == INT32_MAX) ? -1 : first;
      }
    }
    if (!rlk::temperature_valid(t)) {
      s.r = 0.0f;
      s.l = NAN;
      s.aux = -1;
    }
    if (gr < g.n_rows && h == 0) ws[gr * g.n_sum + n_t] = s;
  }
}

__host__ __device__ __forceinline__ int64_t virtual_blocks(const Geo& g) {
  const int64_t groups = g.m_groups * g.n_groups;
  return ((groups + kXcds - 1) / kXcds) * kXcds * kGM * kGN;
}

// First tile at or after virtual workgroup v (stepping by the grid), or false.
__device__ __forceinline__ bool next_tile(const Geo& g, int64_t n_virtual, int64_t& v, int64_t& m_t, int64_t& n_t) {
  while (v < n_virtual) {
    if (tile_of(g, v, m_t, n_t)) return true;
    v += gridDim.x;
  }
  return false;
}

template <bool kLogp>
__global__ __launch_bounds__(kThreads) void k_linear(Geo g, const float* __restrict__ temperature,
                                                     const int64_t* __restrict__ target,
                                                     ShardSummary* __restrict__ ws, uint16_t* __restrict__ out,
                                                     int64_t ldo) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[kSmem];
  const int64_t n_virtual = virtual_blocks(g);
  const int kt_n = g.d / BK;
  int64_t v = blockIdx.x, m_t = 0, n_t = 0;
  if (!next_tile(g, n_virtual, v, m_t, n_t)) return;  // uniform across the workgroup
  const int lane = threadIdx.x & 63;
  const int wm = (threadIdx.x >> 6) % (BM / kWaveM);
  const int wn = (threadIdx.x >> 6) / (BM / kWaveM);
  Panels p = make_panels(g, m_t * BM, g.col_base + n_t * BN);
  int par = 0;
  bf16x8 fa[kSteps][kMB], fb[kSteps][kNB];
  prefetch_tile(p, kt_n, par, smem);
  // stage 0 landed: all but the last 16 panel loads (stage 1) are done
  asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  load_frags(smem, smem + 2 * kStage, wm, wn, 0, fa[0], fb[0]);
  load_frags(smem, smem + 2 * kStage, wm, wn, 1, fa[1], fb[1]);
  int64_t v2 = v + gridDim.x, m2 = 0, n2 = 0;
  bool more = next_tile(g, n_virtual, v2, m2, n2);
  Panels pn = more ? make_panels(g, m2 * BM, g.col_base + n2 * BN) : p;
  while (true) {
    const int64_t row0 = m_t * BM;
    const int64_t col0 = g.col_base + n_t * BN;
    Acc acc[kMB][kNB];
    tile_logits(g, p, pn, more, par, smem, acc, fa, fb);
    float tr[kMB];
    int64_t tgr[kMB];
    if (kLogp) {
#pragma unroll
      for (int i = 0; i < kMB; ++i) {
        const int64_t gr = row0 + wm * kWaveM + i * 32 + (lane & 31);
        tr[i] = gr < g.n_rows ? temperature[gr] : 1.0f;
        tgr[i] = gr < g.n_rows ? target[gr] : -1;
      }
    }
    if (kLogp)
      tile_summaries(g, row0, col0, acc, tr, tgr, ws);
    else
      tile_store(g, row0, col0, acc, out, ldo);
    if (!more) break;
    par = (par + kt_n) & 1;
    m_t = m2;
    n_t = n2;
    p = pn;
    v = v2;
    v2 = v + gridDim.x;
    more = next_tile(g, n_virtual, v2, m2, n2);
    pn = more ? make_panels(g, m2 * BM, g.col_base + n2 * BN) : p;
    if (kt_n == 1) {
      // a one-stage tile could not load the next one in its loop
      prefetch_tile(p, kt_n, par, smem);
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      load_frags(smem + par * kStage, smem + (2 + par) * kStage, wm, wn, 0, fa[0], fb[0]);
      load_frags(smem + par * kStage, smem + (2 + par) * kStage, wm, wn, 1, fa[1], fb[1]);
    }
  }
  (void)wn;
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

// Compute units of the current device (cached per device; 0 if unknown).
static int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// One workgroup per compute unit (a workgroup's LDS fills one), each looping
// over its tiles: no workgroup launches between tiles. Workgroup b stays on
// XCD b % 8, so its tiles v = b + k * grid keep the XCD of the tile order.
static unsigned grid_for(const Geo& g) {
  const int64_t v = virtual_blocks(g);
  int64_t cap = cu_count();
  cap = cap > 0 ? (cap + kXcds - 1) / kXcds * kXcds : kMaxGrid;
  if (cap > kMaxGrid) cap = kMaxGrid;
  return static_cast<unsigned>(v < cap ? v : cap);
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
