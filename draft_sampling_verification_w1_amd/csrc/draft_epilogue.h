// draft_epilogue.h -- the draft's per-tile epilogue: for one row and one
// 32-token block (lane pair n, n + 32, 16 logits each) the running
// log-sum-exp of z = U_k + B_k and the block's score log-mass + Gumbel
// variate, bracketed by its binary32 error bound, for the first level of the
// two-level Gumbel-max draw from p_k = softmax(z) (summary page §3.1).
#pragma once

#include "device_common.h"

namespace dspark {

__device__ __forceinline__ float sum16(const float* e) {
  float a0 = (e[0] + e[1]) + (e[2] + e[3]);
  float a1 = (e[4] + e[5]) + (e[6] + e[7]);
  float a2 = (e[8] + e[9]) + (e[10] + e[11]);
  float a3 = (e[12] + e[13]) + (e[14] + e[15]);
  return (a0 + a1) + (a2 + a3);
}

__device__ __forceinline__ float max16(const float* z) {
  float a0 = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
  float a1 = fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7]));
  float a2 = fmaxf(fmaxf(z[8], z[9]), fmaxf(z[10], z[11]));
  float a3 = fmaxf(fmaxf(z[12], z[13]), fmaxf(z[14], z[15]));
  return fmaxf(fmaxf(a0, a1), fmaxf(a2, a3));
}

__device__ __forceinline__ void decode16(u32x4 a, u32x4 b, float* out) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    out[2 * i] = bf16_lo(w[i]);
    out[2 * i + 1] = bf16_hi(w[i]);
  }
}

// Running state of one row over a range of blocks.
struct DraftLane {
  float M;        // running max of z
  double S;       // sum of exp(z - M)
  CandState cand;
  u32x4 words;    // Philox block holding the current block's variate
  __device__ void init() {
    M = -INFINITY;
    S = 0.0;
    cand.init();
  }
};

// Logit z[j] = u[j] + b[j] of token 32 t + 16 h + j of row (r, k): u the
// backbone logit (-inf at or beyond V), b the binary32 bias.  `first` marks the
// first block of the lane's range (the Philox block of four block words is
// fetched there and at every fourth block).  dz bounds the contraction error
// of every bias of the block; a log-sum-exp moves by at most its inputs'
// largest error, so it widens the bracket.
//
// Accuracy of the block's log-mass: exponents are taken in base 2 against the
// block maximum mt.  The exponent fma(b, L, fma(u, L, -mt2)) (L = log2 e,
// mt2 = fl(mt L)) is rounded only relative to |z - mt|, never to |z|, and the
// exact residual mt2_lo = mt L - mt2 of the one rounded product is taken out
// once per block: log sum_v e^(z_v) = mt + (log2 s - mt2_lo) ln 2, and the
// block sum enters the running sum as s 2^(-mt2_lo).  What remains is the
// hardware exp2 / log2 error and the 32-term sum (a few 2^-24 relative).
// (One fma on z = fl(u + b) instead saves 16 instructions per block but
// rounds relative to |z|: the lse error at |lse| ~ 20 grows from ~1.5e-7 to
// ~7e-7, most of the 1e-6 margin of the acceptance decisions.)
__device__ __forceinline__ void draft_block_epilogue(DraftLane& st, const float* u, const float* b,
                                                     int r, int k, int t, bool first, uint64_t seed,
                                                     float dz) {
  if (first || (t & 3) == 0) st.words = noise_block(seed, kStreamDraft, r, k, (uint32_t)t >> 2);
  float zm[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) zm[j] = u[j] + b[j];
  const float mt = max_halves(max16(zm));
  if (mt == -INFINITY) return;  // block without mass
  const float mt2 = mt * kLog2e;
  const float mt2_lo = fmaf(mt, kLog2e, -mt2);
  float e[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    e[j] = __builtin_amdgcn_exp2f(fmaf(b[j], kLog2e, fmaf(u[j], kLog2e, -mt2)));
  const float s = sum_halves(sum16(e));
  const float sn = fmaf(s, -mt2_lo * kLn2, s);  // s 2^(-mt2_lo) to first order (|mt2_lo| < 2^-17)
  {
    // one exponential whichever maximum is larger (lanes of a wave differ),
    // the smaller against the larger; st.M = -inf at the first block gives 0
    const bool up = mt > st.M;
    const float f = __builtin_amdgcn_exp2f(-fabsf(st.M - mt) * kLog2e);
    st.S = up ? fma(st.S, (double)f, (double)sn) : fma((double)sn, (double)f, st.S);
    st.M = up ? mt : st.M;
  }
  const float sc = fmaf(__builtin_amdgcn_logf(s) - mt2_lo, kLn2, mt) +
                   gumbel_f32(word_of(st.words, t & 3));
  const float d = fmaf(kScoreRel, fabsf(mt), kScoreAbs) + dz;
  st.cand.add(sc - d, sc + d, t);
}

}  // namespace dspark
