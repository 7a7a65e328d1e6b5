// device_common.h -- gfx950 device primitives for the DSpark hot path:
// counter-based noise, bf16 unpacking, wave64 exchanges and the partial-result
// records the split-vocabulary kernels hand to their merge kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace dspark {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Random-number streams.  A two-level draw takes its block variates from
// stream s and its member variates from stream s + kMemberStream.
constexpr uint32_t kStreamDraft = 0, kStreamAccept = 1, kStreamResidual = 2, kStreamBonus = 3;
constexpr uint32_t kMemberStream = 4;

// Error bound of a binary32 block score (log-mass + Gumbel variate, see
// BlockCands) against its exact value:
//   |score32 - score| <= kScoreAbs + kScoreRel |m| + dz,
// m the block's largest logit.  dz = kContractErr ||W1[x]||_1 max|W2| over
// the tile bounds the contraction error of every logit (zero where no bias is
// added); a log-sum-exp moves by at most its inputs' largest error.  The other
// two terms cover the rest, with wide margins: the rounding of z = U + B
// (2^-24 |z|, whose weighted mean over the block is at most |m| + 12), the
// exp2 arguments and results, the 32-term sum, the log2 and the binary32
// Gumbel transform (each a few 2^-24 relative, at most ~2^-20 absolute).
constexpr float kScoreAbs = 0x1p-12f;
constexpr float kScoreRel = 0x1p-17f;

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies, a word permutation and a key xor; the key advances by
// the Weyl increments between rounds.
// ---------------------------------------------------------------------------
// Three-input xor in one gfx950 v_bitop3_b32 (truth table 0x96); the third
// operand is the wave-uniform round key, read straight from an SGPR.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t key) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(key));
  return r;
}

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 x, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t lo_hi0 = (uint64_t)0xD2511F53u * (uint64_t)x.x;
    const uint64_t lo_hi1 = (uint64_t)0xCD9E8D57u * (uint64_t)x.z;
    u32x4 y;
    y.x = xor3((uint32_t)(lo_hi1 >> 32), x.y, k0);
    y.y = (uint32_t)lo_hi1;
    y.z = xor3((uint32_t)(lo_hi0 >> 32), x.w, k1);
    y.w = (uint32_t)lo_hi0;
    x = y;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return x;
}

// Four words for vocabulary entries 4g .. 4g+3 of row (stream, r, k).
__device__ __forceinline__ u32x4 noise_block(uint64_t seed, uint32_t stream, uint32_t r,
                                             uint32_t k, uint32_t group) {
  u32x4 c;
  c.x = group;
  c.y = k;
  c.z = r;
  c.w = stream;
  return philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
}

__device__ __forceinline__ uint32_t word_of(u32x4 b, int i) {
  return i == 0 ? b.x : (i == 1 ? b.y : (i == 2 ? b.z : b.w));
}

// Uniform ((w>>9) + 1/2) 2^-23, exact in binary32: the top 23 bits become the
// mantissa of f in [1, 2) (one v_alignbit), and f - (1 - 2^-24) is exact.
__device__ __forceinline__ float uniform_f32(uint32_t w) {
  const float f = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w, 9));
  return f - 0x1.fffffep-1f;
}

__device__ __forceinline__ double uniform_f64(uint32_t w) {
  return ((double)(w >> 9) + 0.5) * 0x1p-23;
}

// -ln(u) in binary32 with small relative error everywhere: a short series in
// a = 1 - u (exact here) when u is within 2^-6 of 1, the hardware log2 otherwise.
__device__ __forceinline__ float neg_log_uniform_f32(uint32_t w) {
  const float u = uniform_f32(w);
  const float a = 1.0f - u;
  const float series =
      a * fmaf(a, fmaf(a, fmaf(a, fmaf(a, 0.2f, 0.25f), 0.33333334f), 0.5f), 1.0f);
  const float via_log = -__builtin_amdgcn_logf(u) * kLn2;
  return a < 0x1p-6f ? series : via_log;
}

// Gumbel variate for screening candidates (binary32).
__device__ __forceinline__ float gumbel_f32(uint32_t w) {
  return -__builtin_amdgcn_logf(neg_log_uniform_f32(w)) * kLn2;
}

// Gumbel variate for final decisions (binary64).
__device__ __forceinline__ double gumbel_f64(uint32_t w) {
  return -log(-log(uniform_f64(w)));
}

__device__ __forceinline__ float exp_fast(float x) {  // e^x via the hardware exp2
  return __builtin_amdgcn_exp2f(x * kLog2e);
}

// ---------------------------------------------------------------------------
// bf16 / f32 element access
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

// A thread's 16 elements of a 4,096-element slice [base, base + 4096) of a
// row read by a 256-thread workgroup: 16-byte groups at base + E tid + 256 E g
// (E = elements per 16 bytes, g < 16 / E), so that each load instruction of a
// wave covers one contiguous kilobyte.  Entries at or beyond `end` read as
// -inf.  `vec_ok` (row base 16-byte aligned) enables vector loads.
__device__ __forceinline__ void load_slice16(const uint16_t* row, int base, int tid, int end,
                                             bool vec_ok, float* out) {
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int v = base + 8 * tid + 2048 * g;
    if (vec_ok && v + 8 <= end) {
      const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + v));
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[8 * g + 2 * i] = bf16_lo(w[i]);
        out[8 * g + 2 * i + 1] = bf16_hi(w[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) out[8 * g + i] = (v + i < end) ? bf16_at(row, v + i) : -INFINITY;
    }
  }
}

__device__ __forceinline__ void load_slice16(const float* row, int base, int tid, int end,
                                             bool vec_ok, float* out) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int v = base + 4 * tid + 1024 * g;
    if (vec_ok && v + 4 <= end) {
      const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + v));
      out[4 * g] = q.x;
      out[4 * g + 1] = q.y;
      out[4 * g + 2] = q.z;
      out[4 * g + 3] = q.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) out[4 * g + i] = (v + i < end) ? row[v + i] : -INFINITY;
    }
  }
}

__device__ __forceinline__ float elem_at(const uint16_t* p, int64_t i) { return bf16_at(p, i); }
__device__ __forceinline__ float elem_at(const float* p, int64_t i) { return p[i]; }

// ---------------------------------------------------------------------------
// Online log-sum-exp state and Gumbel-argmax candidates.
// ---------------------------------------------------------------------------
struct LseState {
  float m;   // running maximum (binary32 values seen)
  double s;  // sum of exp(x - m)
};

__device__ __forceinline__ void lse_init(LseState& st) {
  st.m = -INFINITY;
  st.s = 0.0;
}

// Merge two (m, s) pairs in binary64.
__device__ __forceinline__ void lse_merge(float& m, double& s, float m2, double s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    s = s2;
    return;
  }
  if (m2 > m) {
    s = s * exp((double)m - (double)m2) + s2;
    m = m2;
  } else {
    s = s + s2 * exp((double)m2 - (double)m);
  }
}

// Candidate order: larger score wins; equal scores -> lower index.
__device__ __forceinline__ bool cand_better(double s1, int i1, double s2, int i2) {
  return (s1 > s2) || (s1 == s2 && (unsigned)i1 < (unsigned)i2);
}

// Lane exchange across the two halves of a wave64.
template <typename T>
__device__ __forceinline__ T xor32(T v) {
  return __shfl_xor(v, 32, 64);
}

// Lane l combined with lane l ^ 32 in one v_permlane32_swap (a VALU op, no LDS
// round trip).  Given the same value twice, the builtin returns the lower
// half's values in every lane of its first result and the upper half's in its
// second, so the pair is {x[l], x[l ^ 32]} in some order; max and sum are
// symmetric, so every lane gets the same bits as with xor32.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// Partial records written per (vocabulary split, row) and merged later.
// Arrays are structure-of-arrays with row stride `ld` (the row capacity).
// ---------------------------------------------------------------------------
// Running block-candidate record of a split (see BlockCands).
struct CandState {
  float lo, hi1, hi2;
  int b1;
  __device__ void init() {
    lo = hi1 = hi2 = -INFINITY;
    b1 = -1;
  }
  __device__ void add(float lo_b, float hi_b, int b) {
    lo = fmaxf(lo, lo_b);
    if (hi_b > hi1) {
      hi2 = hi1;
      hi1 = hi_b;
      b1 = b;
    } else {
      hi2 = fmaxf(hi2, hi_b);
    }
  }
  // Merge another split-part's record (disjoint blocks).
  __device__ void merge(const CandState& o) {
    lo = fmaxf(lo, o.lo);
    if (o.hi1 > hi1 || (o.hi1 == hi1 && o.b1 >= 0 && (b1 < 0 || o.b1 < b1))) {
      hi2 = fmaxf(hi1, o.hi2);
      hi1 = o.hi1;
      b1 = o.b1;
    } else {
      hi2 = fmaxf(hi2, o.hi1);
    }
  }
  __device__ void store(const BlockCands& c, int64_t o) const {
    c.lo[o] = lo;
    c.hi1[o] = hi1;
    c.b1[o] = b1;
    c.hi2[o] = hi2;
  }
};

struct LsePartials {
  float* m;
  double* s;
};

struct CandPartials {
  double* score;  // refined binary64 score, -inf if none
  int32_t* idx;   // token id, -1 if none
  double* aux;    // mode dependent: draft z at the candidate
};

}  // namespace dspark
