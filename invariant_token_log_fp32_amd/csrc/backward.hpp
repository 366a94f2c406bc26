// Gradient of the token logprobs with respect to the BF16 logits.
//
// Passages: RL-Kernel page "H100 canonical CP backward validation", Change
// section (the training step back-propagates through the logprobs; the
// observed nonzero gradients came from the KL term), and page "Configurable
// H100 consistency runs", mode/KL paragraph (the KL reference logprob is over
// the full temperature-scaled vocabulary; the policy logprob keeps its
// top-p/top-k support).
//
// For a row with temperature T > 0, target t and upstream gradients g_r (of
// the reference logprob) and g_p (of the policy logprob):
//   d/dx_j = ( [j == t] (g_r + g_p) - g_r p_j - g_p [x_j >= thr] q_j ) / T
// with p_j = 2^(x_j c - lse log2 e) and q_j = 2^(x_j c - lse_S log2 e),
// c = fl32(log2(e) / T), taking lse and lse_S from the forward pass. g_p is
// dropped when the target lies outside the support (the policy logprob is
// the constant -inf there). The target column is formed from the forward's
// logprobs as (g_r (-expm1(ref)) + g_p (-expm1(pol))) / T so that 1 - p_t
// keeps its relative accuracy when p_t is close to 1.
//
// The rows are cut into chunks of 4096 16-byte vectors (32768 columns); a
// 1024-thread workgroup takes one (row, chunk) item at a time, issues all of
// its 16-byte non-temporal loads of 8 BF16 logits at once (4 per lane), then
// computes and writes the 16-byte non-temporal stores of 8 BF16 gradients
// (rounded to nearest even); pad columns are written as 0. Items run in
// row-major order, so the workgroups resident at any moment read and write a
// narrow window of consecutive memory, which keeps the mixed read/write
// stream close to the HBM copy rate. Each output element depends only on its
// own row's inputs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "logp_device.hpp"
#include "rlk_logp.h"

namespace rlk {

constexpr int kBwdThreads = 1024;
constexpr int kBwdUnroll = 4;                              // vectors in flight per lane
constexpr int64_t kBwdChunk = int64_t(kBwdThreads) * kBwdUnroll;  // vectors per work item

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to packed BF16 (round to nearest even; NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

struct BwdRow {
  float c;      // fl32(log2(e) / T)
  float a_r;    // -lse * log2(e)
  float s_r;    // -g_r / T
  float a_p;    // -lse_S * log2(e)
  float s_p;    // -g_p / T (0 when the policy term is absent)
  float thr;    // support threshold on the BF16 value
  float g_t;    // value of the target column
  int64_t vt;   // vector holding the target column
  int et;       // its position in the vector
};

// Gradient of the 8 columns of one vector (all real columns).
template <bool kPolicy>
__device__ __forceinline__ void grad8(const u32x4& v, const BwdRow& R, float (&g)[8]) {
  float x[8];
  unpack8(v, x);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const float e = __builtin_amdgcn_exp2f(fmaf(x[u], R.c, R.a_r));
    float gu = R.s_r * e;
    if (kPolicy) {
      const float q = (x[u] >= R.thr) ? __builtin_amdgcn_exp2f(fmaf(x[u], R.c, R.a_p)) : 0.0f;
      gu = gu + R.s_p * q;
    }
    g[u] = gu;
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&g)[8]) {
  u32x4 o;
  o.x = pack_bf16x2(g[0], g[1]);
  o.y = pack_bf16x2(g[2], g[3]);
  o.z = pack_bf16x2(g[4], g[5]);
  o.w = pack_bf16x2(g[6], g[7]);
  return o;
}

// One chunk [v0, v1) of a row's 16-byte vectors: vectors below
// ceil(vocab_real / 8) hold real columns (the last one possibly only in
// part), the rest are pad.
template <bool kPolicy>
__device__ __forceinline__ void grad_chunk(const uint16_t* __restrict__ rowp, uint16_t* __restrict__ outp,
                                           int64_t vocab_real, int64_t v0, int64_t v1, const BwdRow& R) {
  const int64_t nv_real = (vocab_real + 7) / 8;
  const int64_t lim = v1 < nv_real ? v1 : nv_real;
  const u32x4* __restrict__ src = reinterpret_cast<const u32x4*>(rowp);
  u32x4* __restrict__ dst = reinterpret_cast<u32x4*>(outp);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 in[kBwdUnroll];
#pragma unroll
  for (int u = 0; u < kBwdUnroll; ++u) {
    const int64_t v = v0 + u * kBwdThreads + threadIdx.x;
    in[u] = zero;
    if (v < lim) in[u] = __builtin_nontemporal_load(src + v);
  }
#pragma unroll
  for (int u = 0; u < kBwdUnroll; ++u) {
    const int64_t v = v0 + u * kBwdThreads + threadIdx.x;
    if (v >= v1) break;
    if (v >= nv_real) {
      __builtin_nontemporal_store(zero, dst + v);
      continue;
    }
    float g[8];
    grad8<kPolicy>(in[u], R, g);
    if (v == R.vt) {
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = (e == R.et) ? R.g_t : g[e];
    }
    if ((v + 1) * 8 > vocab_real) {  // the vector holding the last real column
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = (v * 8 + e < vocab_real) ? g[e] : 0.0f;
    }
    __builtin_nontemporal_store(pack8(g), dst + v);
  }
}

// Fills the real columns of vectors [v0, v1) with `real` (a BF16 pattern
// pair) and the pad columns with 0.
__device__ __forceinline__ void fill_chunk(uint16_t* __restrict__ outp, int64_t vocab_real, int64_t v0, int64_t v1,
                                           uint32_t real) {
  u32x4* __restrict__ dst = reinterpret_cast<u32x4*>(outp);
  for (int64_t v = v0 + threadIdx.x; v < v1; v += kBwdThreads) {
    uint32_t w[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int64_t col = v * 8 + 2 * h;
      const uint32_t lo = (col < vocab_real) ? (real & 0xFFFFu) : 0u;
      const uint32_t hi = (col + 1 < vocab_real) ? (real & 0xFFFF0000u) : 0u;
      w[h] = lo | hi;
    }
    const u32x4 o = {w[0], w[1], w[2], w[3]};
    __builtin_nontemporal_store(o, dst + v);
  }
}

}  // namespace rlk
