// bias_pass.hip -- split-vocabulary passes over (request, position) rows that
// need the Markov-head bias B = W1[x_{k-1}] W2 (rank 256) added to the
// backbone logits U:
//   draft    : online log-sum-exp of z = U + B and the Gumbel-argmax candidate
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
// row, so the epilogue reads U (and T) with two 16-byte loads per lane; those
// loads are issued one tile ahead.  Binary32 rows compute the same bias with a
// VALU dot product.
//
// Draft candidates are screened without a Gumbel transform per token: with
// e_i = exp(z_i - m) (already needed for the softmax sum) and L_i = log2 u_i,
// token i beats the lane's current best b iff L_i * e_b > e_i * L_b, which is
// z_i - ln(-ln u_i) > z_b - ln(-ln u_b) rearranged.  Only the lane's final
// candidate gets its score in binary64.
//
// Workgroup = 8 waves x 32 rows; grid = (vocabulary splits, row blocks).
#include "device_common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kWaves = 8;
constexpr int kRowsPerBlock = kWaves * 32;
constexpr int kThreads = kWaves * 64;

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

// 16 consecutive elements [v, v+16) of a row in storage form; entries at or
// beyond V hold -inf.
template <typename E>
struct Frag;

template <>
struct Frag<uint16_t> {
  u32x4 a, b;
};

template <>
struct Frag<float> {
  f32x4 q[4];
};

__device__ __forceinline__ Frag<uint16_t> frag_load(const uint16_t* row, int v, int V, bool vec_ok) {
  Frag<uint16_t> f;
  if (row == nullptr) {
    f.a = f.b = (u32x4){0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};
  } else if (vec_ok && v + 16 <= V) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row + v);
    f.a = __builtin_nontemporal_load(p);
    f.b = __builtin_nontemporal_load(p + 1);
  } else {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t lo = (v + 2 * i < V) ? row[v + 2 * i] : 0xFF80u;
      const uint32_t hi = (v + 2 * i + 1 < V) ? row[v + 2 * i + 1] : 0xFF80u;
      w[i] = lo | (hi << 16);
    }
    f.a = (u32x4){w[0], w[1], w[2], w[3]};
    f.b = (u32x4){w[4], w[5], w[6], w[7]};
  }
  return f;
}

__device__ __forceinline__ Frag<float> frag_load(const float* row, int v, int V, bool vec_ok) {
  Frag<float> f;
  if (row != nullptr && vec_ok && v + 16 <= V) {
    const f32x4* p = reinterpret_cast<const f32x4*>(row + v);
#pragma unroll
    for (int i = 0; i < 4; ++i) f.q[i] = __builtin_nontemporal_load(p + i);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 q;
      q.x = (row && v + 4 * i + 0 < V) ? row[v + 4 * i + 0] : -INFINITY;
      q.y = (row && v + 4 * i + 1 < V) ? row[v + 4 * i + 1] : -INFINITY;
      q.z = (row && v + 4 * i + 2 < V) ? row[v + 4 * i + 2] : -INFINITY;
      q.w = (row && v + 4 * i + 3 < V) ? row[v + 4 * i + 3] : -INFINITY;
      f.q[i] = q;
    }
  }
  return f;
}

__device__ __forceinline__ void frag_decode(const Frag<uint16_t>& f, float* out) {
  const uint32_t w[8] = {f.a.x, f.a.y, f.a.z, f.a.w, f.b.x, f.b.y, f.b.z, f.b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    out[2 * i] = bf16_lo(w[i]);
    out[2 * i + 1] = bf16_hi(w[i]);
  }
}

__device__ __forceinline__ void frag_decode(const Frag<float>& f, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[4 * i] = f.q[i].x;
    out[4 * i + 1] = f.q[i].y;
    out[4 * i + 2] = f.q[i].z;
    out[4 * i + 3] = f.q[i].w;
  }
}

// Staged rows: 32 rows x 64 tokens of bf16 per wave, rows padded to 144 bytes
// so the 16-byte fragment reads of 32 rows spread over the LDS banks.
constexpr int kRowStride = 144;

// 8 consecutive bf16 [v, v+8) of a row (one 16-byte load when aligned and in
// range); -inf for entries at or beyond V and for rows that are not active.
__device__ __forceinline__ u32x4 chunk_load(const uint16_t* row, int v, int V, bool vec_ok) {
  if (row == nullptr) return (u32x4){0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};
  if (vec_ok && v + 8 <= V) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + v));
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (v + 2 * i < V) ? row[v + 2 * i] : 0xFF80u;
    const uint32_t hi = (v + 2 * i + 1 < V) ? row[v + 2 * i + 1] : 0xFF80u;
    w[i] = lo | (hi << 16);
  }
  return (u32x4){w[0], w[1], w[2], w[3]};
}

template <int MODE>
struct LaneState;

template <>
struct LaneState<kModeDraft> {
  float m;     // running max of z
  double s;    // sum of exp(z - m)
  float Lb;    // log2 u of the candidate (< 0; -1 before the first one)
  float eb;    // exp(z - m) of the candidate (0 before the first one)
  float bacc;  // bias at the candidate
  int idx;
  __device__ void init() {
    m = -INFINITY;
    s = 0.0;
    Lb = -1.0f;
    eb = 0.0f;
    bacc = 0.0f;
    idx = -1;
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

// Per-tile epilogue: the lane holds the bias acc[j] of tokens vb + j (j < 16)
// of one row, with that row's backbone logits u[j] (and target logits t[j]).
template <int MODE>
__device__ __forceinline__ void epilogue(LaneState<MODE>& st, const float* acc, const float* u,
                                         const float* t, const RowCtx& rc, int vb, int V,
                                         uint64_t seed) {
  if constexpr (MODE == kModeDraft) {
    float z[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = u[j] + acc[j];
    float mt = z[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mt = fmaxf(mt, z[j]);
    if (mt > st.m) {
      const float f = (st.m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((st.m - mt) * kLog2e);
      st.s *= (double)f;
      st.eb *= f;
      st.m = mt;
    }
    if (st.m == -INFINITY) return;
    float e[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) e[j] = __builtin_amdgcn_exp2f((z[j] - st.m) * kLog2e);
    st.s += (double)sum16(e);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (vb + 4 * q < V) {
        const u32x4 w = noise_block(seed, kStreamDraft, rc.r, rc.k, (uint32_t)(vb >> 2) + q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * q + i;
          const float L = __builtin_amdgcn_logf(uniform_f32(word_of(w, i)));
          const bool better = fmaf(L, st.eb, -e[j] * st.Lb) > 0.0f;
          st.Lb = better ? L : st.Lb;
          st.eb = better ? e[j] : st.eb;
          st.bacc = better ? acc[j] : st.bacc;
          st.idx = better ? vb + j : st.idx;
        }
      }
    }
  } else if constexpr (MODE == kModeCstar) {
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
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * q + i;
          if (vb + j < V) {
            const uint32_t wd = word_of(w, i);
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

template <typename E>
__device__ __forceinline__ float row_elem(const void* row, int v) {
  return elem_at(reinterpret_cast<const E*>(row), v);
}

// Final binary64 scoring of the lane's candidate, merge of the two wave halves
// (which hold the same rows) and the partial record written by the lower half.
template <int MODE, typename E>
__device__ __forceinline__ void finish(const LaneState<MODE>& st, const RowCtx& rc, int row,
                                       int split, const BiasPassArgs& a, bool writer) {
  const int64_t o = (int64_t)row * a.nsplit + split;
  if constexpr (MODE == kModeDraft) {
    double sc = -INFINITY, z = 0.0;
    if (rc.active && st.idx >= 0) {
      z = (double)row_elem<E>(rc.urow, st.idx) + (double)st.bacc;
      const u32x4 w = noise_block(a.seed, kStreamDraft, rc.r, rc.k, (uint32_t)st.idx >> 2);
      sc = z + gumbel_f64(word_of(w, st.idx & 3));
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
__global__ __launch_bounds__(kThreads) void k_bias_bf16(const BiasPassArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int active_rows = a.row_count ? min(*a.row_count, a.nrows) : a.nrows;
  const int row0 = blockIdx.y * kRowsPerBlock;
  if (row0 >= active_rows) return;
  const int split = blockIdx.x;
  const int t0 = (int)((int64_t)split * a.ntiles / a.nsplit);
  const int t1 = (int)((int64_t)(split + 1) * a.ntiles / a.nsplit);
  const bool vec_ok = a.vec_ok != 0;
  constexpr bool kNeedT = MODE != kModeDraft;

  const int row = row0 + wave * 32 + n;
  const RowCtx rc = row_ctx(a, row, active_rows, true);
  bf16x8 bop[kSteps];
  if (rc.active) {
    const u32x4* w1 = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint16_t*>(a.W1) + (int64_t)rc.prev * kRank + 128 * h);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) bop[s] = as_bf16x8(w1[s]);
  } else {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) bop[s] = as_bf16x8((u32x4){0u, 0u, 0u, 0u});
  }
  LaneState<MODE> st;
  st.init();
  const uint16_t* urow = rc.active ? reinterpret_cast<const uint16_t*>(rc.urow) : nullptr;
  const uint16_t* trow = (rc.active && kNeedT) ? reinterpret_cast<const uint16_t*>(rc.trow) : nullptr;

  // Each wave streams the packed W2 tile itself (1 KB contiguous per load
  // instruction, shared by the workgroup's waves through L2), so waves never
  // wait on each other and one wave's MFMAs overlap another's epilogue.
  //
  // U (and T) rows are staged per wave in 64-token chunks: each load
  // instruction covers 8 rows x 128 contiguous bytes (whole cache lines), the
  // lanes then read their MFMA-layout fragment (row n, 16 tokens) from the
  // wave's own LDS region.  Per-lane 32-byte fragment loads straight from HBM
  // (32 rows per instruction) stream at under half that bandwidth.  The next
  // chunk's loads are in flight while the current chunk's two tiles compute.
  constexpr int kNS = kNeedT ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t lds_rows[kWaves][kNS][32 * kRowStride];
  uint8_t* my_u = lds_rows[wave][0];
  uint8_t* my_t = lds_rows[wave][kNS - 1];
  const int lr = lane >> 3;          // row within a group of 8
  const int lc = (lane & 7) * 8;     // token offset within the chunk
  const uint16_t* ld_u[4];
  const uint16_t* ld_t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ld_u[i] = reinterpret_cast<const uint16_t*>(
        __shfl((unsigned long long)(uintptr_t)urow, 8 * i + lr, 64));
    ld_t[i] = reinterpret_cast<const uint16_t*>(
        __shfl((unsigned long long)(uintptr_t)trow, 8 * i + lr, 64));
  }
  const u32x4* W2p = reinterpret_cast<const u32x4*>(a.W2p) + lane;
  u32x4 ru[4], rt[4];
  const int nt = t1 - t0;
  if (nt > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ru[i] = chunk_load(ld_u[i], t0 * kTile + lc, a.V, vec_ok);
      if (kNeedT) rt[i] = chunk_load(ld_t[i], t0 * kTile + lc, a.V, vec_ok);
    }
  }
  for (int c = 0; 2 * c < nt; ++c) {
    const int tt = t0 + 2 * c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(my_u + (8 * i + lr) * kRowStride + 2 * lc) = ru[i];
      if (kNeedT) *reinterpret_cast<u32x4*>(my_t + (8 * i + lr) * kRowStride + 2 * lc) = rt[i];
    }
    __builtin_amdgcn_wave_barrier();
    if (2 * c + 2 < nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ru[i] = chunk_load(ld_u[i], (tt + 2) * kTile + lc, a.V, vec_ok);
        if (kNeedT) rt[i] = chunk_load(ld_t[i], (tt + 2) * kTile + lc, a.V, vec_ok);
      }
    }
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int t = tt + tau;
      if (t >= t1) break;
      const u32x4* At = W2p + (int64_t)t * 1024;
      u32x4 av[kSteps];
#pragma unroll
      for (int s = 0; s < kSteps; ++s) av[s] = At[s * 64];
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < kSteps; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[s]), bop[s], acc, 0, 0, 0);
      if (rc.active) {
        float accv[16], u[16], tv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) accv[j] = acc[j];
        const int off = n * kRowStride + tau * 64 + h * 32;
        Frag<uint16_t> fu;
        fu.a = *reinterpret_cast<const u32x4*>(my_u + off);
        fu.b = *reinterpret_cast<const u32x4*>(my_u + off + 16);
        frag_decode(fu, u);
        if (kNeedT) {
          Frag<uint16_t> ft;
          ft.a = *reinterpret_cast<const u32x4*>(my_t + off);
          ft.b = *reinterpret_cast<const u32x4*>(my_t + off + 16);
          frag_decode(ft, tv);
        }
        epilogue<MODE>(st, accv, u, tv, rc, t * kTile + 16 * h, a.V, a.seed);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  finish<MODE, uint16_t>(st, rc, row, split, a, h == 0);
}

// Binary32 rows: same row/lane layout, bias by VALU dot products against the
// transposed W2 ([ceil(V/32)*32, 256], zero rows beyond V).
template <int MODE>
__global__ __launch_bounds__(kThreads) void k_bias_f32(const BiasPassArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int active_rows = a.row_count ? min(*a.row_count, a.nrows) : a.nrows;
  const int row0 = blockIdx.y * kRowsPerBlock;
  if (row0 >= active_rows) return;
  const int split = blockIdx.x;
  const int t0 = (int)((int64_t)split * a.ntiles / a.nsplit);
  const int t1 = (int)((int64_t)(split + 1) * a.ntiles / a.nsplit);
  const bool vec_ok = a.vec_ok != 0;
  const f32x4* W2T = reinterpret_cast<const f32x4*>(a.W2p);
  constexpr bool kNeedT = MODE != kModeDraft;

  const int row = row0 + wave * 32 + n;
  const RowCtx rc = row_ctx(a, row, active_rows, false);
  LaneState<MODE> st;
  st.init();
  if (rc.active) {
    const f32x4* w1 = reinterpret_cast<const f32x4*>(
        reinterpret_cast<const float*>(a.W1) + (int64_t)rc.prev * kRank);
    for (int t = t0; t < t1; ++t) {
      const int vb = t * kTile + 16 * h;
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
      float u[16], tv[16];
      frag_decode(frag_load(reinterpret_cast<const float*>(rc.urow), vb, a.V, vec_ok), u);
      if (kNeedT) frag_decode(frag_load(reinterpret_cast<const float*>(rc.trow), vb, a.V, vec_ok), tv);
      epilogue<MODE>(st, acc, u, tv, rc, vb, a.V, a.seed);
    }
  }
  finish<MODE, float>(st, rc, row, split, a, h == 0);
}

// One wave per request row: merge the vocabulary splits of position k
// (maximum first, then the rescaled sums, so each partial needs one exp).
__global__ __launch_bounds__(64) void k_draft_merge(int R, int gamma, int k, int nsplit,
                                                    const float* pm, const double* ps,
                                                    const double* cscore, const int32_t* cidx,
                                                    const double* caux, int32_t* tokens,
                                                    double* lse, double* logq) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t base = (int64_t)r * nsplit;
  float M = -INFINITY;
  double sc = -INFINITY;
  int idx = -1, from = -1;
  for (int j = lane; j < nsplit; j += 64) {
    M = fmaxf(M, pm[base + j]);
    const double sc2 = cscore[base + j];
    const int i2 = cidx[base + j];
    if (cand_better(sc2, i2, sc, idx)) {
      sc = sc2;
      idx = i2;
      from = j;
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    M = fmaxf(M, __shfl_xor(M, off, 64));
    const double sc2 = __shfl_xor(sc, off, 64);
    const int i2 = __shfl_xor(idx, off, 64);
    const int f2 = __shfl_xor(from, off, 64);
    if (cand_better(sc2, i2, sc, idx)) {
      sc = sc2;
      idx = i2;
      from = f2;
    }
  }
  double s = 0.0;
  for (int j = lane; j < nsplit; j += 64) {
    const float m = pm[base + j];
    if (m != -INFINITY) s += ps[base + j] * exp((double)m - (double)M);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) {
    const double l = (double)M + log(s);
    const int64_t o = (int64_t)r * gamma + (k - 1);
    tokens[o] = idx;
    lse[o] = l;
    logq[o] = (from >= 0 ? caux[base + from] : 0.0) - l;
  }
}

}  // namespace

// Vocabulary splits: enough workgroups for one full round on MI355X (256 CUs,
// one 8-wave workgroup each), never more splits than 32-token tiles.  Split s
// covers tiles [s*ntiles/nsplit, (s+1)*ntiles/nsplit).
BiasGeometry bias_geometry(int nrows, int V) {
  constexpr int kSlots = 256;
  BiasGeometry g;
  g.rows_per_block = kRowsPerBlock;
  g.row_blocks = (nrows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int ntiles = (V + kTile - 1) / kTile;
  g.nsplit = min(ntiles, max(1, (kSlots + g.row_blocks - 1) / g.row_blocks));
  g.tiles_per_split = (ntiles + g.nsplit - 1) / g.nsplit;
  return g;
}

hipError_t launch_bias_pass(int mode, bool bf16, const BiasPassArgs& a, hipStream_t stream) {
  TimingScope timing(mode == kModeDraft ? "draft_bias" : (mode == kModeCstar ? "cstar_bias" : "residual_bias"), stream);
  const dim3 grid(a.nsplit, (a.nrows + kRowsPerBlock - 1) / kRowsPerBlock);
  const dim3 block(kThreads);
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
  TimingScope timing("draft_merge", stream);
  hipLaunchKernelGGL(k_draft_merge, dim3(R), dim3(64), 0, stream, R, gamma, k, nsplit, pm, ps,
                     cscore, cidx, caux, tokens, lse, logq);
  return hipGetLastError();
}

}  // namespace dspark
