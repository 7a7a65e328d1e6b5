// bias_pass.hip -- split-vocabulary passes over (request, position) rows that
// need the Markov-head bias B = W1[x_{k-1}] W2 (rank 256) added to the
// backbone logits U:
//   draft    : online log-sum-exp of z = U + B and Gumbel-argmax candidates
//              (summary page §3.1: p_k = softmax(U_k + B_k), left-to-right draws)
//   cstar    : sum_v min(p^d_v, p^t_v) = 1 - ||p^d - p^t||_1 / 2 (summary page §3.2.1)
//   residual : Gumbel-argmax over ln max(0, p^t - p^d) at the first rejection,
//              with ln p^t as fallback (standard speculative rejection sampling)
//
// bf16 rows use the gfx950 matrix cores: a 32-token tile of the packed W2 is
// the A operand (staged once per workgroup in LDS, double buffered), the
// gathered W1 rows of 32 rows are the B operand (held in registers for the
// whole pass), v_mfma_f32_32x32x16_bf16 accumulates in fp32.  The packed tile
// order makes each lane's 16 accumulators cover 16 consecutive tokens of one
// row, so the epilogue reads U (and T) with two 16-byte loads per lane.
// Binary32 rows compute the same bias with a VALU dot product.
//
// Workgroup = 4 waves x 64 rows; grid = (vocabulary splits, row blocks).
#include "device_common.h"
#include "kernels.h"

namespace dspark {

namespace {

struct RowCtx {
  bool active;
  int r, k;
  int prev;
  const void* urow;
  const void* trow;
  float ld32, lt32;
  double ld64, lt64;
};

__device__ __forceinline__ RowCtx row_ctx(const BiasPassArgs& a, int i, int active_rows, bool bf16) {
  RowCtx c;
  c.active = i < active_rows;
  c.r = 0;
  c.k = 1;
  c.prev = 0;
  c.urow = nullptr;
  c.trow = nullptr;
  c.ld32 = c.lt32 = 0.f;
  c.ld64 = c.lt64 = 0.0;
  if (!c.active) return c;
  if (a.row_ids) {
    const int id = a.row_ids[i];
    c.r = id / a.gamma;
    c.k = id - c.r * a.gamma + 1;
  } else {
    c.r = i;
    c.k = a.k;
  }
  int x = (c.k == 1) ? a.anchors[c.r] : a.tokens[(int64_t)c.r * a.gamma + (c.k - 2)];
  c.prev = min(max(x, 0), a.V - 1);
  const size_t esz = bf16 ? 2 : 4;
  c.urow = (const char*)a.U + ((int64_t)c.r * a.gamma + (c.k - 1)) * (int64_t)a.V * esz;
  if (a.T) c.trow = (const char*)a.T + ((int64_t)c.r * (a.gamma + 1) + (c.k - 1)) * (int64_t)a.V * esz;
  if (a.lse_d) {
    c.ld64 = a.lse_d[(int64_t)c.r * a.gamma + (c.k - 1)];
    c.ld32 = (float)c.ld64;
  }
  if (a.lse_t) {
    c.lt64 = a.lse_t[(int64_t)c.r * (a.gamma + 1) + (c.k - 1)];
    c.lt32 = (float)c.lt64;
  }
  return c;
}

template <int MODE>
struct LaneState;

template <>
struct LaneState<kModeDraft> {
  float m;
  double s;
  float best;
  int idx;
  float bacc, bu;
  uint32_t bw;
  __device__ void init() {
    m = -INFINITY;
    s = 0.0;
    best = -INFINITY;
    idx = -1;
    bacc = bu = 0.f;
    bw = 0;
  }
};

template <>
struct LaneState<kModeCstar> {
  double s;
  __device__ void init() { s = 0.0; }
};

template <>
struct LaneState<kModeResidual> {
  float best;
  int idx;
  float bacc, bu, bt;
  uint32_t bw;
  float fbest;
  int fidx;
  float ft;
  uint32_t fw;
  __device__ void init() {
    best = fbest = -INFINITY;
    idx = fidx = -1;
    bacc = bu = bt = ft = 0.f;
    bw = fw = 0;
  }
};

__device__ __forceinline__ float sum16(const float* e) {
  float a0 = (e[0] + e[1]) + (e[2] + e[3]);
  float a1 = (e[4] + e[5]) + (e[6] + e[7]);
  float a2 = (e[8] + e[9]) + (e[10] + e[11]);
  float a3 = (e[12] + e[13]) + (e[14] + e[15]);
  return (a0 + a1) + (a2 + a3);
}

// Per-tile epilogue: the lane holds bias acc[j] of tokens vb + j (j < 16) of
// one row.
template <int MODE, typename E>
__device__ __forceinline__ void epilogue(LaneState<MODE>& st, const float* acc, const RowCtx& rc,
                                         int vb, int V, bool vec_ok, uint64_t seed) {
  float u[16];
  load16(reinterpret_cast<const E*>(rc.urow), vb, V, vec_ok, u);
  if constexpr (MODE == kModeDraft) {
    float z[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = u[j] + acc[j];
    float mt = z[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mt = fmaxf(mt, z[j]);
    if (mt > st.m) {
      if (st.m != -INFINITY) st.s *= exp((double)st.m - (double)mt);
      st.m = mt;
    }
    if (st.m != -INFINITY) {
      float e[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) e[j] = __builtin_amdgcn_exp2f((z[j] - st.m) * kLog2e);
      st.s += (double)sum16(e);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (vb + 4 * q < V) {
        const u32x4 w = noise_block(seed, kStreamDraft, rc.r, rc.k, (uint32_t)(vb >> 2) + q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * q + e;
          if (vb + j < V) {
            const uint32_t wd = word_of(w, e);
            const float sc = z[j] + gumbel_f32(wd);
            if (sc > st.best) {
              st.best = sc;
              st.idx = vb + j;
              st.bacc = acc[j];
              st.bu = u[j];
              st.bw = wd;
            }
          }
        }
      }
    }
  } else {
    float t[16];
    load16(reinterpret_cast<const E*>(rc.trow), vb, V, vec_ok, t);
    if constexpr (MODE == kModeCstar) {
      float e[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float lpd = (u[j] - rc.ld32) + acc[j];
        const float lpt = t[j] - rc.lt32;
        e[j] = __builtin_amdgcn_exp2f(fminf(lpd, lpt) * kLog2e);
      }
      st.s += (double)sum16(e);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (vb + 4 * q < V) {
          const u32x4 w = noise_block(seed, kStreamResidual, rc.r, rc.k, (uint32_t)(vb >> 2) + q);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 4 * q + e;
            if (vb + j < V) {
              const uint32_t wd = word_of(w, e);
              const float g = gumbel_f32(wd);
              const float lpt = t[j] - rc.lt32;
              const float sf = lpt + g;
              if (sf > st.fbest) {
                st.fbest = sf;
                st.fidx = vb + j;
                st.ft = t[j];
                st.fw = wd;
              }
              const float lpd = (u[j] - rc.ld32) + acc[j];
              const float d = lpd - lpt;
              if (d < 0.f) {
                const float sc = lpt + logf(-expm1f(d)) + g;
                if (sc > st.best) {
                  st.best = sc;
                  st.idx = vb + j;
                  st.bacc = acc[j];
                  st.bu = u[j];
                  st.bt = t[j];
                  st.bw = wd;
                }
              }
            }
          }
        }
      }
    }
  }
}

// Refine the lane's candidate in binary64, merge the two wave halves (which
// hold the same rows) and let the lower half write the partial record.
template <int MODE>
__device__ __forceinline__ void finish(const LaneState<MODE>& st, const RowCtx& rc, int row,
                                       int split, const BiasPassArgs& a, bool writer) {
  const int64_t o = (int64_t)row * a.nsplit + split;
  if constexpr (MODE == kModeDraft) {
    double sc = -INFINITY, z = 0.0;
    if (st.idx >= 0) {
      z = (double)st.bu + (double)st.bacc;
      sc = z + gumbel_f64(st.bw);
    }
    float m = st.m;
    double s = st.s;
    int idx = st.idx;
    const float m2 = xor32(m);
    const double s2 = xor32(s);
    const double sc2 = xor32(sc);
    const int i2 = xor32(idx);
    const double z2 = xor32(z);
    lse_merge(m, s, m2, s2);
    if (cand_better(sc2, i2, sc, idx)) {
      sc = sc2;
      idx = i2;
      z = z2;
    }
    if (writer && rc.active) {
      a.pm[o] = m;
      a.ps[o] = s;
      a.cscore[o] = sc;
      a.cidx[o] = idx;
      a.caux[o] = z;
    }
  } else if constexpr (MODE == kModeCstar) {
    const double s = st.s + xor32(st.s);
    if (writer && rc.active) a.ps[o] = s;
  } else {
    double sc = -INFINITY, sf = -INFINITY;
    if (st.idx >= 0) {
      const double lpd = ((double)st.bu + (double)st.bacc) - rc.ld64;
      const double lpt = (double)st.bt - rc.lt64;
      const double d = lpd - lpt;
      if (d < 0.0) sc = lpt + log(-expm1(d)) + gumbel_f64(st.bw);
    }
    if (st.fidx >= 0) sf = ((double)st.ft - rc.lt64) + gumbel_f64(st.fw);
    int idx = st.idx, fidx = st.fidx;
    const double sc2 = xor32(sc), sf2 = xor32(sf);
    const int i2 = xor32(idx), f2 = xor32(fidx);
    if (cand_better(sc2, i2, sc, idx)) {
      sc = sc2;
      idx = i2;
    }
    if (cand_better(sf2, f2, sf, fidx)) {
      sf = sf2;
      fidx = f2;
    }
    if (writer && rc.active) {
      a.cscore[o] = sc;
      a.cidx[o] = (sc > -INFINITY) ? idx : -1;
      a.fscore[o] = sf;
      a.fidx[o] = fidx;
    }
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int MODE>
__global__ __launch_bounds__(256) void k_bias_bf16(const BiasPassArgs a) {
  __shared__ u32x4 lds_a[2][kSteps * 64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int active_rows = a.row_count ? min(*a.row_count, a.nrows) : a.nrows;
  const int row0 = blockIdx.y * 256;
  if (row0 >= active_rows) return;
  const int split = blockIdx.x;
  const int t0 = split * a.tiles_per_split;
  const int t1 = min(t0 + a.tiles_per_split, a.ntiles);
  const bool vec_ok = a.vec_ok != 0;

  RowCtx rc[2];
  bf16x8 bop[2][kSteps];
  LaneState<MODE> st[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int i = row0 + wave * 64 + nb * 32 + n;
    rc[nb] = row_ctx(a, i, active_rows, true);
    st[nb].init();
    if (rc[nb].active) {
      const u32x4* w1 = reinterpret_cast<const u32x4*>(
          reinterpret_cast<const uint16_t*>(a.W1) + (int64_t)rc[nb].prev * kRank + 128 * h);
#pragma unroll
      for (int s = 0; s < kSteps; ++s) bop[nb][s] = as_bf16x8(w1[s]);
    } else {
#pragma unroll
      for (int s = 0; s < kSteps; ++s) bop[nb][s] = as_bf16x8((u32x4){0u, 0u, 0u, 0u});
    }
  }

  const u32x4* W2p = reinterpret_cast<const u32x4*>(a.W2p);
  if (t0 < t1) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      lds_a[0][threadIdx.x + 256 * q] = W2p[(int64_t)t0 * 1024 + threadIdx.x + 256 * q];
  }
  __syncthreads();
  for (int t = t0; t < t1; ++t) {
    const int buf = (t - t0) & 1;
    const bool has_next = t + 1 < t1;
    u32x4 pre[4];
    if (has_next) {
#pragma unroll
      for (int q = 0; q < 4; ++q) pre[q] = W2p[(int64_t)(t + 1) * 1024 + threadIdx.x + 256 * q];
    }
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const bf16x8 av = as_bf16x8(lds_a[buf][s * 64 + lane]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bop[0][s], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bop[1][s], acc1, 0, 0, 0);
    }
    const int vb = t * kTile + 16 * h;
    float accv[16];
    if (rc[0].active) {
#pragma unroll
      for (int j = 0; j < 16; ++j) accv[j] = acc0[j];
      epilogue<MODE, uint16_t>(st[0], accv, rc[0], vb, a.V, vec_ok, a.seed);
    }
    if (rc[1].active) {
#pragma unroll
      for (int j = 0; j < 16; ++j) accv[j] = acc1[j];
      epilogue<MODE, uint16_t>(st[1], accv, rc[1], vb, a.V, vec_ok, a.seed);
    }
    if (has_next) {
#pragma unroll
      for (int q = 0; q < 4; ++q) lds_a[buf ^ 1][threadIdx.x + 256 * q] = pre[q];
    }
    __syncthreads();
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
    finish<MODE>(st[nb], rc[nb], row0 + wave * 64 + nb * 32 + n, split, a, h == 0);
}

// Binary32 rows: same row/lane layout, bias by VALU dot products against the
// transposed W2 ([ceil(V/32)*32, 256], zero rows beyond V).
template <int MODE>
__global__ __launch_bounds__(256) void k_bias_f32(const BiasPassArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int active_rows = a.row_count ? min(*a.row_count, a.nrows) : a.nrows;
  const int row0 = blockIdx.y * 256;
  if (row0 >= active_rows) return;
  const int split = blockIdx.x;
  const int t0 = split * a.tiles_per_split;
  const int t1 = min(t0 + a.tiles_per_split, a.ntiles);
  const bool vec_ok = a.vec_ok != 0;
  const f32x4* W2T = reinterpret_cast<const f32x4*>(a.W2p);

  RowCtx rc[2];
  LaneState<MODE> st[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    rc[nb] = row_ctx(a, row0 + wave * 64 + nb * 32 + n, active_rows, false);
    st[nb].init();
  }
  for (int t = t0; t < t1; ++t) {
    const int vb = t * kTile + 16 * h;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      if (!rc[nb].active) continue;
      const f32x4* w1 = reinterpret_cast<const f32x4*>(
          reinterpret_cast<const float*>(a.W1) + (int64_t)rc[nb].prev * kRank);
      float acc[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = 0.f;
      for (int i4 = 0; i4 < kRank / 4; ++i4) {
        const f32x4 x = w1[i4];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const f32x4 y = W2T[(int64_t)(vb + j) * (kRank / 4) + i4];
          acc[j] = fmaf(x.x, y.x, acc[j]);
          acc[j] = fmaf(x.y, y.y, acc[j]);
          acc[j] = fmaf(x.z, y.z, acc[j]);
          acc[j] = fmaf(x.w, y.w, acc[j]);
        }
      }
      epilogue<MODE, float>(st[nb], acc, rc[nb], vb, a.V, vec_ok, a.seed);
    }
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
    finish<MODE>(st[nb], rc[nb], row0 + wave * 64 + nb * 32 + n, split, a, h == 0);
}

// One wave per request row: merge the vocabulary splits of position k.
__global__ __launch_bounds__(64) void k_draft_merge(int R, int gamma, int k, int nsplit,
                                                    const float* pm, const double* ps,
                                                    const double* cscore, const int32_t* cidx,
                                                    const double* caux, int32_t* tokens,
                                                    double* lse, double* logq) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  float m = -INFINITY;
  double s = 0.0, sc = -INFINITY, z = 0.0;
  int idx = -1;
  for (int j = lane; j < nsplit; j += 64) {
    const int64_t o = (int64_t)r * nsplit + j;
    lse_merge(m, s, pm[o], ps[o]);
    const double sc2 = cscore[o];
    const int i2 = cidx[o];
    if (cand_better(sc2, i2, sc, idx)) {
      sc = sc2;
      idx = i2;
      z = caux[o];
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const double s2 = __shfl_xor(s, off, 64);
    const double sc2 = __shfl_xor(sc, off, 64);
    const int i2 = __shfl_xor(idx, off, 64);
    const double z2 = __shfl_xor(z, off, 64);
    lse_merge(m, s, m2, s2);
    if (cand_better(sc2, i2, sc, idx)) {
      sc = sc2;
      idx = i2;
      z = z2;
    }
  }
  if (lane == 0) {
    const double l = (double)m + log(s);
    const int64_t o = (int64_t)r * gamma + (k - 1);
    tokens[o] = idx;
    lse[o] = l;
    logq[o] = z - l;
  }
}

}  // namespace

BiasGeometry bias_geometry(int nrows, int V) {
  BiasGeometry g;
  g.rows_per_block = 256;
  g.row_blocks = (nrows + 255) / 256;
  const int ntiles = (V + kTile - 1) / kTile;
  const int target = max(1, (512 + g.row_blocks - 1) / g.row_blocks);
  g.tiles_per_split = max(1, (ntiles + target - 1) / target);
  g.nsplit = (ntiles + g.tiles_per_split - 1) / g.tiles_per_split;
  return g;
}

hipError_t launch_bias_pass(int mode, bool bf16, const BiasPassArgs& a, hipStream_t stream) {
  const dim3 grid(a.nsplit, (a.nrows + 255) / 256);
  const dim3 block(256);
  if (bf16) {
    if (mode == kModeDraft) hipLaunchKernelGGL(k_bias_bf16<kModeDraft>, grid, block, 0, stream, a);
    else if (mode == kModeCstar) hipLaunchKernelGGL(k_bias_bf16<kModeCstar>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(k_bias_bf16<kModeResidual>, grid, block, 0, stream, a);
  } else {
    if (mode == kModeDraft) hipLaunchKernelGGL(k_bias_f32<kModeDraft>, grid, block, 0, stream, a);
    else if (mode == kModeCstar) hipLaunchKernelGGL(k_bias_f32<kModeCstar>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(k_bias_f32<kModeResidual>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_draft_merge(int R, int gamma, int k, int nsplit, const float* pm,
                              const double* ps, const double* cscore, const int32_t* cidx,
                              const double* caux, int32_t* tokens, double* lse, double* logq,
                              hipStream_t stream) {
  hipLaunchKernelGGL(k_draft_merge, dim3(R), dim3(64), 0, stream, R, gamma, k, nsplit, pm, ps,
                     cscore, cidx, caux, tokens, lse, logq);
  return hipGetLastError();
}

}  // namespace dspark
