// select_impl.h -- device code of the binary64 second stage of the two-level
// Gumbel-max draws, as a workgroup-level function (one row per call).  See
// select.hip for the method.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace dspark {
namespace sel {

constexpr int kMaxCand = 1024;

// Position of tile-local token j among the 32 lanes of a packed W2 tile (the
// inverse of the tile's token permutation).
__device__ __forceinline__ int packed_slot(int j) {
  return (j & 3) | ((j >> 4) << 2) | (((j >> 2) & 3) << 3);
}

// Partial bias sum_{i in [32p, 32p+32)} w1[i] W2[i][v] in binary64, eight
// threads per token, as two steps so that the loads of a block (and of its
// stored logits) are all in flight before any arithmetic waits on them.
struct BiasLoad {
  u32x4 c[8];  // bf16: 4 packed-tile chunks; binary32: 8 chunks of the row
};

__device__ __forceinline__ void bias64_load(BiasLoad& L, const void* W2p, bool bf16, int v, int p) {
  if (bf16) {
    const u32x4* tile = reinterpret_cast<const u32x4*>(W2p) + (int64_t)(v >> 5) * (kSteps * 64);
    const int m = packed_slot(v & 31);
    const int hh = p >> 2, s0 = (p & 3) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) L.c[i] = tile[(s0 + i) * 64 + 32 * hh + m];
  } else {
    const u32x4* rowp = reinterpret_cast<const u32x4*>(W2p) + (int64_t)v * (kRank / 4) + 8 * p;
#pragma unroll
    for (int i = 0; i < 8; ++i) L.c[i] = rowp[i];
  }
}

__device__ __forceinline__ double bias64_dot(const BiasLoad& L, bool bf16, const double* w1, int p) {
  double acc = 0.0;
  if (bf16) {
    const int hh = p >> 2, s0 = (p & 3) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double* w = w1 + 128 * hh + 8 * (s0 + i);
      acc = fma(w[0], (double)bf16_lo(L.c[i].x), acc);
      acc = fma(w[1], (double)bf16_hi(L.c[i].x), acc);
      acc = fma(w[2], (double)bf16_lo(L.c[i].y), acc);
      acc = fma(w[3], (double)bf16_hi(L.c[i].y), acc);
      acc = fma(w[4], (double)bf16_lo(L.c[i].z), acc);
      acc = fma(w[5], (double)bf16_hi(L.c[i].z), acc);
      acc = fma(w[6], (double)bf16_lo(L.c[i].w), acc);
      acc = fma(w[7], (double)bf16_hi(L.c[i].w), acc);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double* w = w1 + 32 * p + 4 * i;
      acc = fma(w[0], (double)__uint_as_float(L.c[i].x), acc);
      acc = fma(w[1], (double)__uint_as_float(L.c[i].y), acc);
      acc = fma(w[2], (double)__uint_as_float(L.c[i].z), acc);
      acc = fma(w[3], (double)__uint_as_float(L.c[i].w), acc);
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

// Block-wide max of four values / sum of one (blockDim.x = 64 * nw, nw <= 8);
// every thread gets the results.
__device__ void block_max4(double* x, double (*sh)[8]) {
  const int nw = blockDim.x >> 6;
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
  for (int c = 0; c < 4; ++c) {
    double m = sh[c][0];
    for (int w = 1; w < nw; ++w) m = fmax(m, sh[c][w]);
    x[c] = m;
  }
  __syncthreads();
}

__device__ double block_sum(double x, double (*sh)[8]) {
  const int nw = blockDim.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[0][threadIdx.x >> 6] = x;
  __syncthreads();
  double r = sh[0][0];
  for (int w = 1; w < nw; ++w) r += sh[0][w];
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

// Log-weight of a token of the draw from its stored logits (u: U, t: T) and
// its bias (draft, residual).
template <int MODE>
__device__ __forceinline__ double log_weight(bool fallback, const SelRow& q, double u, double t,
                                             double bias) {
  if constexpr (MODE == kSelDraft) {
    return u + bias;
  } else if constexpr (MODE == kSelBonus) {
    return t;
  } else {
    const double lpt = t - q.lt;
    if (fallback) return lpt;
    const double lpd = u + bias - q.ld;
    return lpt > lpd ? lpt + log1p(-exp(lpd - lpt)) : -INFINITY;
  }
}

// Split records held per thread: split j lives in thread j % nt, slot j / nt.
// Draft and residual passes have at most 256 splits (one per thread), the
// bonus pass up to 2048.
template <int MODE>
struct RecSlots {
  static constexpr int K = MODE == kSelBonus ? 8 : 1;
};

// Workgroup-shared state of one row's select.
struct SelShared {
  double w1s[kRank];
  double red[4][8];
  int cand[kMaxCand];
  int ncand, overflow;
  double zc[32], gc[32];  // scored block: log-weights and member Gumbel variates
  double zb[32], gb[32];  // best block so far
  int bstar, brun;        // winning block; best block after the latest scoring
  u32x4 rows[32 * 32];    // draft: W1 rows of the best block's tokens (16-byte chunks)
};

// The draw of row i (draft: request i at position a.k; residual / bonus: entry
// i of the work list).  blockDim.x = 256.
template <int MODE>
__device__ void select_row(const SelectArgs& a, int bf16_flag, int i, SelShared& sh, int kpos) {
  constexpr int K = RecSlots<MODE>::K;
  constexpr bool kDraft = MODE == kSelDraft;
  constexpr bool kResid = MODE == kSelResidual;
  constexpr bool kBias = MODE != kSelBonus;
  double* const w1s = sh.w1s;
  double (*red)[8] = sh.red;
  const bool bf16 = bf16_flag != 0;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;

  SelRow q;
  q.rec = i;
  q.ld = q.lt = 0.0;
  q.uoff = q.toff = 0;
  q.prev = 0;
  if constexpr (kDraft) {
    q.r = i;
    q.k = kpos;
  } else {
    if (i >= *a.row_count) return;
    const int id = a.row_ids[i];
    if constexpr (kResid) {
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
    q.uoff = ((int64_t)q.r * a.gamma + (q.k - 1)) * a.V;
    if (kDraft && a.bop_in != nullptr) {
      // the previous select left W1[x_{k-1}] as this row's B operands: one load
      // instead of the token and then its row
      if (tid < kRank) {
        const int c = tid >> 3;  // 16-byte chunk c = 16h + s holds elements [8c, 8c + 8)
        const uint16_t* chunk = reinterpret_cast<const uint16_t*>(a.bop_in) + bop_chunk(q.r, c & 15, c >> 4) * 8;
        w1s[tid] = (double)bf16_at(chunk, tid & 7);
      }
    } else {
      const int x = (q.k == 1) ? a.anchors[q.r] : a.tokens[(int64_t)q.r * a.gamma + (q.k - 2)];
      q.prev = min(max(x, 0), a.V - 1);
      if (tid < kRank) w1s[tid] = stored(a.W1, bf16, (int64_t)q.prev * kRank + tid);
    }
  }
  const int64_t rec0 = (int64_t)q.rec * a.nsplit;
  const uint32_t sblock = kDraft ? kStreamDraft : (kResid ? kStreamResidual : kStreamBonus);

  // 1. every field of the thread's split records in one batch of loads
  float pm[K], lo[K], h1[K], h2[K], lof[K], h1f[K], h2f[K];
  double ps[K];
  int b1[K], b1f[K];
  double wsum = 0.0;
#pragma unroll
  for (int s = 0; s < K; ++s) {
    const int j = tid + s * nt;
    const bool has = j < a.nsplit;
    const int64_t o = rec0 + (has ? j : 0);
    pm[s] = lo[s] = h1[s] = h2[s] = lof[s] = h1f[s] = h2f[s] = -INFINITY;
    ps[s] = 0.0;
    b1[s] = b1f[s] = -1;
    if (has) {
      lo[s] = a.cand.lo[o];
      h1[s] = a.cand.hi1[o];
      h2[s] = a.cand.hi2[o];
      b1[s] = a.cand.b1[o];
      if constexpr (kDraft) {
        pm[s] = a.pm[o];
        ps[s] = a.ps[o];
      }
      if constexpr (kResid) {
        lof[s] = a.cand_f.lo[o];
        h1f[s] = a.cand_f.hi1[o];
        h2f[s] = a.cand_f.hi2[o];
        b1f[s] = a.cand_f.b1[o];
        wsum += (double)a.wpos[o];
      }
    }
  }

  // 2. max logit (draft), largest lower bounds of both record sets, residual
  //    mass (residual)
  double mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int s = 0; s < K; ++s) {
    mx[0] = fmax(mx[0], (double)pm[s]);
    mx[1] = fmax(mx[1], (double)lo[s]);
    mx[2] = fmax(mx[2], (double)lof[s]);
  }
  block_max4(mx, red);
  double lse = 0.0;
  if constexpr (kDraft) {
    double S = 0.0;
#pragma unroll
    for (int s = 0; s < K; ++s)
      if (pm[s] != -INFINITY) S += ps[s] * exp((double)pm[s] - mx[0]);
    S = block_sum(S, red);
    lse = mx[0] + log(S);
  }
  bool fallback = false;
  if constexpr (kResid) fallback = !(block_sum(wsum, red) > 0.0);

  const int tj = tid >> 3, tp = tid & 7;
  // draft: the W1 rows of a scored block's tokens are fetched with it, so that
  // the drafted token's row can be written out as the next position's B
  // operand without another round trip
  const bool pre_rows = kDraft && a.bop_out != nullptr;
  int bstar = -1;
  for (int attempt = 0; attempt < 2 && bstar < 0; ++attempt) {
    if (attempt == 1) {
      if (!kResid || fallback) break;
      fallback = true;  // no block of the residual has binary64 mass: p^t instead
    }
    const bool useF = kResid && fallback;
    const double Ls = useF ? mx[2] : mx[1];
    // 3. blocks whose upper bound reaches the largest lower bound
    if (tid == 0) {
      sh.ncand = 0;
      sh.overflow = 0;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < K; ++s) {
      const int j = tid + s * nt;
      const double hh1 = useF ? h1f[s] : h1[s];
      const double hh2 = useF ? h2f[s] : h2[s];
      const int bb1 = useF ? b1f[s] : b1[s];
      if (j < a.nsplit && hh2 > -INFINITY && hh2 >= Ls) {
        const int t0 = split_tile(j, a.nsplit, a.ntiles, a.tiles_per_stage);
        const int t1 = split_tile(j + 1, a.nsplit, a.ntiles, a.tiles_per_stage);
        const int pos = atomicAdd(&sh.ncand, t1 - t0);
        if (pos + (t1 - t0) <= kMaxCand) {
          for (int t = t0; t < t1; ++t) sh.cand[pos + t - t0] = t;
        } else {
          sh.overflow = 1;
        }
      } else if (j < a.nsplit && hh1 > -INFINITY && hh1 >= Ls && bb1 >= 0) {
        const int pos = atomicAdd(&sh.ncand, 1);
        if (pos < kMaxCand) sh.cand[pos] = bb1;
        else sh.overflow = 1;
      }
    }
    __syncthreads();
    const bool all = sh.overflow != 0;
    const int total = all ? a.ntiles : min(sh.ncand, kMaxCand);
    // 4. binary64 score of each such block: eight threads per token for the
    //    bias; the token's stored logits, W2 chunks and member Gumbel variate
    //    are fetched and computed together, then one wave takes the block's
    //    log-mass and Gumbel variate
    double best = -INFINITY;
    int bb = -1;
    for (int ci = 0; ci < total; ++ci) {
      const int blk = all ? ci : sh.cand[ci];
      const int v = blk * kTile + tj;
      const bool tok = tid < 256 && v < a.V;
      BiasLoad L;
      if (kBias && tok) bias64_load(L, a.W2p, bf16, v, tp);
      u32x4 wrow[4];
      if (pre_rows && tok) {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.W1) + (int64_t)v * (kRank / 8) + 4 * tp;
#pragma unroll
        for (int c = 0; c < 4; ++c) wrow[c] = src[c];
      }
      double u = 0.0, t = 0.0;
      if (tok && tp == 0) {
        if constexpr (MODE != kSelBonus) u = stored(a.U, bf16, q.uoff + v);
        if constexpr (MODE != kSelDraft) t = stored(a.T, bf16, q.toff + v);
      }
      const double g = (tok && tp == 1) ? gumbel_at(a.seed, sblock + kMemberStream, q.r, q.k, (uint32_t)v) : 0.0;
      double part = (kBias && tok) ? bias64_dot(L, bf16, w1s, tp) : 0.0;
      part += __shfl_xor(part, 1, 64);
      part += __shfl_xor(part, 2, 64);
      part += __shfl_xor(part, 4, 64);
      if (tid < 256 && tp == 0) sh.zc[tj] = tok ? log_weight<MODE>(fallback, q, u, t, part) : -INFINITY;
      if (tid < 256 && tp == 1) sh.gc[tj] = g;
      __syncthreads();
      if (tid < 32) {
        const double w = sh.zc[tid];
        double m = w;
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) m = fmax(m, __shfl_xor(m, off, 64));
        if (total == 1) {
          // the only block that can win: its score decides nothing
          if (m > -INFINITY) {
            bb = blk;
            sh.zb[tid] = w;
            sh.gb[tid] = sh.gc[tid];
          }
        } else {
          double s = (m > -INFINITY) ? exp(w - m) : 0.0;
#pragma unroll
          for (int off = 1; off < 32; off <<= 1) s += __shfl_xor(s, off, 64);
          if (m > -INFINITY) {
            const double sc = m + log(s) + gumbel_at(a.seed, sblock, q.r, q.k, (uint32_t)blk);
            if (bb < 0 || sc > best || (sc == best && blk < bb)) {
              best = sc;
              bb = blk;
              sh.zb[tid] = w;
              sh.gb[tid] = sh.gc[tid];
            }
          }
        }
        if (tid == 0) sh.brun = bb;
      }
      __syncthreads();
      if (pre_rows && tok && sh.brun == blk) {
#pragma unroll
        for (int c = 0; c < 4; ++c) sh.rows[tj * 32 + 4 * tp + c] = wrow[c];
      }
    }
    if (tid == 0) sh.bstar = bb;
    __syncthreads();
    bstar = sh.bstar;
    __syncthreads();
  }

  // 5. member of the winning block (its log-weights and variates are in zb, gb)
  if (tid < 32) {
    int x = -1;
    double wx = -INFINITY;
    if (bstar >= 0) {
      const int v = bstar * kTile + tid;
      const double w = sh.zb[tid];
      const double sc = (w > -INFINITY) ? w + sh.gb[tid] : -INFINITY;
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
    if (pre_rows) {
      // lane c writes chunk c of the row of max(x, 0) (the next pass clamps
      // the previous token the same way)
      const int c = tid;
      const u32x4 val = x >= 0 ? sh.rows[(x - bstar * kTile) * 32 + c]
                               : reinterpret_cast<const u32x4*>(a.W1)[c];
      reinterpret_cast<u32x4*>(a.bop_out)[bop_chunk(q.r, c & 15, c >> 4)] = val;
    }
    if (tid == 0) {
      if constexpr (kDraft) {
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


}  // namespace sel
}  // namespace dspark
