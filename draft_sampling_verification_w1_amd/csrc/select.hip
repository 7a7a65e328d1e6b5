// select.hip -- binary64 second stage of the two-level Gumbel-max draws: the
// draft token of position k (summary page §3.1), the corrective token drawn
// from max(0, p^t - p^d) at the first rejection and the bonus token drawn from
// p^t after full acceptance (standard speculative rejection sampling, notes
// page 배경).
//
// A draw picks a 32-entry block by Gumbel-max over the blocks' log-masses, then
// a member of that block by Gumbel-max over its log-weights; exact ties go to
// the lowest block / entry.  The split passes leave, per (row, split), the
// bracket [lo, hi] of every block's binary32 score in compressed form (largest
// lo, best hi with its block, second-best hi).  One workgroup per row here:
//   1. merges the splits (draft: log-sum-exp of the logits);
//   2. L* = largest lower bound over all blocks; only a block whose upper bound
//      reaches L* can win, so each split contributes its best block if hi1 >= L*,
//      or all of its blocks if hi2 >= L* too;
//   3. rescores those blocks in binary64 from the stored inputs (the bias
//      recomputed from W1 and the packed W2) and keeps the best;
//   4. draws the member of the winning block in binary64.
#include "device_common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kSelThreads = 256;
constexpr int kMaxCand = 1024;

// Position of tile-local token j among the 32 lanes of a packed W2 tile (the
// inverse of the tile's token permutation).
__device__ __forceinline__ int packed_slot(int j) {
  return (j & 3) | ((j >> 4) << 2) | (((j >> 2) & 3) << 3);
}

// Partial bias sum_{i in [32p, 32p+32)} w1[i] W2[i][v] in binary64 (eight
// threads per token; four independent 16-byte loads of the packed tile).
__device__ double bias64_part(const void* W2p, bool bf16, const double* w1, int v, int p) {
  double acc = 0.0;
  if (bf16) {
    const u32x4* tile = reinterpret_cast<const u32x4*>(W2p) + (int64_t)(v >> 5) * (kSteps * 64);
    const int m = packed_slot(v & 31);
    const int hh = p >> 2, s0 = (p & 3) * 4;
    u32x4 c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = tile[(s0 + i) * 64 + 32 * hh + m];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double* w = w1 + 128 * hh + 8 * (s0 + i);
      acc = fma(w[0], (double)bf16_lo(c[i].x), acc);
      acc = fma(w[1], (double)bf16_hi(c[i].x), acc);
      acc = fma(w[2], (double)bf16_lo(c[i].y), acc);
      acc = fma(w[3], (double)bf16_hi(c[i].y), acc);
      acc = fma(w[4], (double)bf16_lo(c[i].z), acc);
      acc = fma(w[5], (double)bf16_hi(c[i].z), acc);
      acc = fma(w[6], (double)bf16_lo(c[i].w), acc);
      acc = fma(w[7], (double)bf16_hi(c[i].w), acc);
    }
  } else {
    const f32x4* rowp = reinterpret_cast<const f32x4*>(W2p) + (int64_t)v * (kRank / 4) + 8 * p;
    f32x4 c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = rowp[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double* w = w1 + 32 * p + 4 * i;
      acc = fma(w[0], (double)c[i].x, acc);
      acc = fma(w[1], (double)c[i].y, acc);
      acc = fma(w[2], (double)c[i].z, acc);
      acc = fma(w[3], (double)c[i].w, acc);
    }
  }
  return acc;
}

__device__ __forceinline__ double stored(const void* p, bool bf16, int64_t i) {
  return bf16 ? (double)bf16_at(reinterpret_cast<const uint16_t*>(p), i)
              : (double)reinterpret_cast<const float*>(p)[i];
}

__device__ __forceinline__ double gumbel_at(uint64_t seed, uint32_t stream, int r, int k, uint32_t v) {
  const u32x4 b = noise_block(seed, stream, (uint32_t)r, (uint32_t)k, v >> 2);
  return gumbel_f64(word_of(b, v & 3));
}

// Block-wide (256 threads) max of four values / sum of one, every thread gets
// the results.
__device__ void block_max4(double* x, double (*sh)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x[c] = fmax(x[c], __shfl_xor(x[c], off, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int c = 0; c < 4; ++c) sh[c][threadIdx.x >> 6] = x[c];
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 4; ++c) x[c] = fmax(fmax(sh[c][0], sh[c][1]), fmax(sh[c][2], sh[c][3]));
  __syncthreads();
}

__device__ double block_sum(double x, double (*sh)[4]) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[0][threadIdx.x >> 6] = x;
  __syncthreads();
  const double r = (sh[0][0] + sh[0][1]) + (sh[0][2] + sh[0][3]);
  __syncthreads();
  return r;
}

struct SelRow {
  int rec;        // record row (index into the split records)
  int r, k;       // request and 1-based position of the draw's random numbers
  int prev;       // previous token (draft, residual)
  int64_t uoff;   // element offset of the U row (draft, residual)
  int64_t toff;   // element offset of the T row (residual, bonus)
  double ld, lt;  // residual: lse of p^d and p^t
};

// Log-weight of token v (< V) of the draw, given its bias (draft, residual).
template <int MODE>
__device__ __forceinline__ double log_weight(const SelectArgs& a, bool bf16, bool fallback,
                                             const SelRow& q, double bias, int v) {
  if constexpr (MODE == kSelDraft) {
    return stored(a.U, bf16, q.uoff + v) + bias;
  } else if constexpr (MODE == kSelBonus) {
    return stored(a.T, bf16, q.toff + v);
  } else {
    const double lpt = stored(a.T, bf16, q.toff + v) - q.lt;
    if (fallback) return lpt;
    const double lpd = stored(a.U, bf16, q.uoff + v) + bias - q.ld;
    return lpt > lpd ? lpt + log1p(-exp(lpd - lpt)) : -INFINITY;
  }
}

template <int MODE>
__global__ __launch_bounds__(kSelThreads) void k_select(const SelectArgs a, int bf16_flag) {
  __shared__ double w1s[kRank];
  __shared__ double red[4][4];
  __shared__ int cand[kMaxCand];
  __shared__ int ncand, overflow;
  __shared__ double zc[32], zb[32];  // log-weights of the scored block and of the best block
  __shared__ int bstar_sh;
  const bool bf16 = bf16_flag != 0;
  const int tid = threadIdx.x;
  const int i = blockIdx.x;
  constexpr bool kBias = MODE != kSelBonus;

  SelRow q;
  q.rec = i;
  q.ld = q.lt = 0.0;
  q.uoff = q.toff = 0;
  q.prev = 0;
  if constexpr (MODE == kSelDraft) {
    q.r = i;
    q.k = a.k;
  } else {
    if (i >= *a.row_count) return;
    const int id = a.row_ids[i];
    if constexpr (MODE == kSelResidual) {
      q.r = id / a.gamma;
      q.k = id - q.r * a.gamma + 1;
      q.toff = ((int64_t)q.r * (a.gamma + 1) + (q.k - 1)) * a.V;
      q.ld = a.lse_d[(int64_t)q.r * a.gamma + (q.k - 1)];
      q.lt = a.lse_t[(int64_t)q.r * (a.gamma + 1) + (q.k - 1)];
    } else {
      q.r = id / (a.gamma + 1);
      q.k = id - q.r * (a.gamma + 1) + 1;
      q.toff = (int64_t)id * a.V;
    }
  }
  if constexpr (kBias) {
    const int x = (q.k == 1) ? a.anchors[q.r] : a.tokens[(int64_t)q.r * a.gamma + (q.k - 2)];
    q.prev = min(max(x, 0), a.V - 1);
    q.uoff = ((int64_t)q.r * a.gamma + (q.k - 1)) * a.V;
    w1s[tid] = stored(a.W1, bf16, (int64_t)q.prev * kRank + tid);
  }
  const int64_t rec0 = (int64_t)q.rec * a.nsplit;
  const uint32_t sblock = MODE == kSelDraft ? kStreamDraft : (MODE == kSelResidual ? kStreamResidual : kStreamBonus);

  // 1. one pass over the split records: max logit (draft), largest lower
  //    bounds of both record sets, residual mass (residual)
  double mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  double wsum = 0.0;
  for (int j = tid; j < a.nsplit; j += kSelThreads) {
    if constexpr (MODE == kSelDraft) mx[0] = fmax(mx[0], (double)a.pm[rec0 + j]);
    mx[1] = fmax(mx[1], (double)a.cand.lo[rec0 + j]);
    if constexpr (MODE == kSelResidual) {
      mx[2] = fmax(mx[2], (double)a.cand_f.lo[rec0 + j]);
      wsum += (double)a.wpos[rec0 + j];
    }
  }
  block_max4(mx, red);
  double lse = 0.0;
  if constexpr (MODE == kSelDraft) {
    double S = 0.0;
    for (int j = tid; j < a.nsplit; j += kSelThreads) {
      const float m = a.pm[rec0 + j];
      if (m != -INFINITY) S += a.ps[rec0 + j] * exp((double)m - mx[0]);
    }
    S = block_sum(S, red);
    lse = mx[0] + log(S);
  }
  bool fallback = false;
  if constexpr (MODE == kSelResidual) fallback = !(block_sum(wsum, red) > 0.0);

  int bstar = -1;
  for (int attempt = 0; attempt < 2 && bstar < 0; ++attempt) {
    if (attempt == 1) {
      if (MODE != kSelResidual || fallback) break;
      fallback = true;  // no block of the residual has binary64 mass: p^t instead
    }
    const BlockCands C = (MODE == kSelResidual && fallback) ? a.cand_f : a.cand;
    const double Ls = (MODE == kSelResidual && fallback) ? mx[2] : mx[1];
    // 2. blocks whose upper bound reaches the largest lower bound
    if (tid == 0) {
      ncand = 0;
      overflow = 0;
    }
    __syncthreads();
    for (int j = tid; j < a.nsplit; j += kSelThreads) {
      const double h1 = C.hi1[rec0 + j], h2 = C.hi2[rec0 + j];
      const int b1 = C.b1[rec0 + j];
      if (h2 > -INFINITY && h2 >= Ls) {
        const int t0 = split_tile(j, a.nsplit, a.ntiles, a.tiles_per_stage);
        const int t1 = split_tile(j + 1, a.nsplit, a.ntiles, a.tiles_per_stage);
        const int pos = atomicAdd(&ncand, t1 - t0);
        if (pos + (t1 - t0) <= kMaxCand) {
          for (int t = t0; t < t1; ++t) cand[pos + t - t0] = t;
        } else {
          overflow = 1;
        }
      } else if (h1 > -INFINITY && h1 >= Ls && b1 >= 0) {
        const int pos = atomicAdd(&ncand, 1);
        if (pos < kMaxCand) cand[pos] = b1;
        else overflow = 1;
      }
    }
    __syncthreads();
    const bool all = overflow != 0;
    const int total = all ? a.ntiles : min(ncand, kMaxCand);
    // 3. binary64 score of each such block: 8 threads per token for the bias,
    //    then one wave takes the block's log-mass and Gumbel variate
    const int tj = tid >> 3, tp = tid & 7;
    double best = -INFINITY;
    int bb = -1;
    for (int ci = 0; ci < total; ++ci) {
      const int blk = all ? ci : cand[ci];
      const int v = blk * kTile + tj;
      double part = 0.0;
      if (kBias && v < a.V) part = bias64_part(a.W2p, bf16, w1s, v, tp);
      part += __shfl_xor(part, 1, 64);
      part += __shfl_xor(part, 2, 64);
      part += __shfl_xor(part, 4, 64);
      if (tp == 0) zc[tj] = v < a.V ? log_weight<MODE>(a, bf16, fallback, q, part, v) : -INFINITY;
      __syncthreads();
      if (tid < 32) {
        const double w = zc[tid];
        double m = w;
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) m = fmax(m, __shfl_xor(m, off, 64));
        double s = (m > -INFINITY) ? exp(w - m) : 0.0;
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) s += __shfl_xor(s, off, 64);
        if (m > -INFINITY) {
          const double sc = m + log(s) + gumbel_at(a.seed, sblock, q.r, q.k, (uint32_t)blk);
          if (bb < 0 || sc > best || (sc == best && blk < bb)) {
            best = sc;
            bb = blk;
            zb[tid] = w;
          }
        }
      }
      __syncthreads();
    }
    if (tid == 0) bstar_sh = bb;
    __syncthreads();
    bstar = bstar_sh;
    __syncthreads();
  }

  // 4. member of the winning block (its log-weights are in zb)
  if (tid < 32) {
    int x = -1;
    double wx = -INFINITY;
    if (bstar >= 0) {
      const int v = bstar * kTile + tid;
      const double w = zb[tid];
      const double sc = (w > -INFINITY) ? w + gumbel_at(a.seed, sblock + kMemberStream, q.r, q.k, (uint32_t)v)
                                        : -INFINITY;
      double bsc = sc;
      int bv = sc > -INFINITY ? v : -1;
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) {
        const double s2 = __shfl_xor(bsc, off, 64);
        const int v2 = __shfl_xor(bv, off, 64);
        if (v2 >= 0 && (bv < 0 || s2 > bsc || (s2 == bsc && v2 < bv))) {
          bsc = s2;
          bv = v2;
        }
      }
      x = bv;
      wx = __shfl(w, x >= 0 ? x - bstar * kTile : 0, 64);
    }
    if (tid == 0) {
      if constexpr (MODE == kSelDraft) {
        const int64_t o = (int64_t)q.r * a.gamma + (q.k - 1);
        a.out_tokens[o] = x;
        a.out_lse[o] = lse;
        a.out_logq[o] = wx - lse;
      } else {
        a.out_tokens[q.r] = x;
      }
    }
  }
}

}  // namespace

hipError_t launch_select(int mode, bool bf16, const SelectArgs& a, hipStream_t stream) {
  const int flag = bf16 ? 1 : 0;
  if (mode == kSelDraft) {
    TimingScope timing("draft_select", stream);
    hipLaunchKernelGGL(k_select<kSelDraft>, dim3(a.R), dim3(kSelThreads), 0, stream, a, flag);
  } else if (mode == kSelResidual) {
    TimingScope timing("residual_select", stream);
    hipLaunchKernelGGL(k_select<kSelResidual>, dim3(a.R), dim3(kSelThreads), 0, stream, a, flag);
  } else {
    TimingScope timing("bonus_select", stream);
    hipLaunchKernelGGL(k_select<kSelBonus>, dim3(a.R), dim3(kSelThreads), 0, stream, a, flag);
  }
  return hipGetLastError();
}

}  // namespace dspark
