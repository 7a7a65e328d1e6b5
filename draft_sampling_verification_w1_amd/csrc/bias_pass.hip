// bias_pass.hip -- split-vocabulary passes over (request, position) rows that
// need the Markov-head bias B = W1[x_{k-1}] W2 (rank 256) added to the
// backbone logits U:
//   draft    : online log-sum-exp of z = U + B, and for every 32-token block
//              its log-mass plus its Gumbel variate -- the first level of the
//              two-level Gumbel-max draw from p_k = softmax(U_k + B_k)
//              (summary page §3.1, left-to-right sampling of the block)
//   cstar    : sum_v min(p^d_v, p^t_v) = 1 - ||p^d - p^t||_1 / 2 (summary page §3.2.1)
//   residual : per block, the mass of max(0, p^t - p^d) and of p^t (the
//              empty-residual fallback), each with its Gumbel variate
//              (standard speculative rejection sampling, notes page 배경)
//
// bf16 rows use the gfx950 matrix cores.  A workgroup owns 256 rows (8 waves x
// 32 rows) and a contiguous range of 32-token tiles, taken two tiles (64
// tokens) per pipeline stage.  Each wave prefetches two stages ahead into
// registers and writes a stage to LDS just before it is used: the packed W2
// tiles (the MFMA A operand, shared by all 8 waves, so each W2 byte crosses
// L2 -> CU once per workgroup) and 128-byte segments of the wave's own rows of
// U (and T), placed with an xor swizzle so that the lanes' 16-byte fragment
// reads hit distinct LDS banks.  The gathered W1 rows of a wave's 32 rows are
// the B operand, held in registers for the whole pass; v_mfma_f32_32x32x16_bf16
// accumulates in fp32.  The packed tile order
// makes lane (n, h) own tokens [16h, 16h+16) of row n, so a 32-token block is
// the lane pair (n, n+32).  In the draft and residual passes the chain
// accumulates B from zero and the backbone logits are added to its result, so
// that the binary32 error of z is bounded by the contraction's own magnitude
// (see kContractErr); the c* pass, which brackets nothing, seeds the
// accumulator with them.  The c* and residual passes read U and T with the
// nontemporal hint (streamed once).  At most 32 rows (bf16) the draft runs
// k_bias_small instead: 4-wave workgroups on tile-granular splits, each wave
// streaming its own tiles with no LDS staging.
// Binary32 rows compute the same bias with a VALU dot product.
#include "device_common.h"
#include "draft_epilogue.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kWaves = 8;
constexpr int kRowsPerBlock = kWaves * 32;
static_assert(kRowsPerBlock == 256, "active_split_count assumes 256-row blocks");
constexpr int kThreads = kWaves * 64;
constexpr int kTileBytesA = kSteps * 64 * 16;  // one packed W2 tile (16 KB)

// s_waitcnt immediate for "at most n vector-memory loads outstanding" (gfx9
// encoding: vmcnt in bits [3:0] and [15:14]; expcnt and lgkmcnt left free).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Workgroup barrier of the stage loop: LDS stores complete, then s_barrier.
// __syncthreads' release fence would also wait for the register prefetches of
// later stages that are still in flight.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Slot swizzle of row n's 16-byte segments within a stage (NSEG segments).
template <int NSEG>
__device__ __forceinline__ int seg_swz(int n) {
  if constexpr (NSEG == 8) return (n ^ (n >> 3)) & 7;
  else return (n >> 1) & 3;
}

struct RowCtx {
  bool active;
  int r, k;
  int prev;
  const void* urow;
  const void* trow;
  float ld2, lt2;  // log2(e) * lse of p^d and p^t
  float eps;       // residual: relative error bound of the binary32 p^d, p^t
};

__device__ __forceinline__ RowCtx row_ctx(const BiasPassArgs& a, int i, int active_rows, bool bf16,
                                          int kpos, bool need_prev = true) {
  RowCtx c;
  c.active = i < active_rows;
  c.r = 0;
  c.k = 1;
  c.prev = 0;
  c.urow = nullptr;
  c.trow = nullptr;
  c.ld2 = c.lt2 = 0.f;
  c.eps = 0.f;
  if (!c.active) return c;
  if (a.row_ids) {
    const int id = a.row_ids[i];
    c.r = id / a.gamma;
    c.k = id - c.r * a.gamma + 1;
  } else {
    c.r = i;
    c.k = kpos;
  }
  if (need_prev) {
    const int32_t* tp = a.tokens + (int64_t)c.r * a.gamma + (c.k - 2);
    const int x = (c.k == 1) ? a.anchors[c.r] : *tp;
    c.prev = min(max(x, 0), a.V - 1);
  }
  const size_t esz = bf16 ? 2 : 4;
  c.urow = (const char*)a.U + ((int64_t)c.r * a.gamma + (c.k - 1)) * (int64_t)a.V * esz;
  if (a.T) c.trow = (const char*)a.T + ((int64_t)c.r * (a.gamma + 1) + (c.k - 1)) * (int64_t)a.V * esz;
  float ld = 0.f, lt = 0.f;
  if (a.lse_d) ld = (float)a.lse_d[(int64_t)c.r * a.gamma + (c.k - 1)];
  if (a.lse_t) lt = (float)a.lse_t[(int64_t)c.r * (a.gamma + 1) + (c.k - 1)];
  c.ld2 = ld * kLog2e;
  c.lt2 = lt * kLog2e;
  c.eps = 0x1p-15f + 0x1p-21f * (fabsf(ld) + fabsf(lt));
  return c;
}

// 8 consecutive bf16 [v, v+8) of a row; -inf for entries at or beyond V and
// for a null row.  Scalar loads (rows that are not 16-byte aligned).
__device__ __forceinline__ u32x4 chunk_load(const uint16_t* row, int v, int V) {
  if (row == nullptr) return (u32x4){0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (v + 2 * i < V) ? row[v + 2 * i] : 0xFF80u;
    const uint32_t hi = (v + 2 * i + 1 < V) ? row[v + 2 * i + 1] : 0xFF80u;
    w[i] = lo | (hi << 16);
  }
  return (u32x4){w[0], w[1], w[2], w[3]};
}

// Eight bf16 -inf: the load source of row segments beyond V and of rows that
// are not active, so that the loaded value needs no select.
__device__ __attribute__((aligned(16))) const uint32_t kNegInfBf16x8[4] = {0xFF80FF80u, 0xFF80FF80u,
                                                                            0xFF80FF80u, 0xFF80FF80u};

typedef __attribute__((address_space(1))) const u32x4 global_u32x4;

// 16-byte load through a global-address-space pointer (a pointer that went
// through a lane shuffle is otherwise a flat access).
__device__ __forceinline__ u32x4 gload16(const void* p) {
  return *(global_u32x4*)(p);
}
// The same with the nontemporal hint: rows read once (measured on MI355X: the
// c* and residual passes, which stream both U and T, gain ~3%; the draft,
// which streams U beside the re-read W2 tiles, does not).
__device__ __forceinline__ u32x4 gload16_nt(const void* p) {
  return __builtin_nontemporal_load((global_u32x4*)(p));
}

// max|W2| of tile t (t uniform across the wave), read through the scalar
// cache.  A vector load here would count against vmcnt behind the stage
// prefetch: since that counter retires in order, waiting for the value before
// each tile's epilogue would drain every stage still in flight.
__device__ __forceinline__ float tile_absmax(const float* tmax, int t) {
  return ((const __attribute__((address_space(4))) float*)tmax)[__builtin_amdgcn_readfirstlane(t)];
}

// ||W1[x]||_1 of a binary32 row (64 16-byte chunks).
__device__ __forceinline__ float w1_norm1(const f32x4* w1) {
  float n1 = 0.f;
  for (int i = 0; i < kRank / 4; ++i) {
    const f32x4 x = w1[i];
    n1 += (fabsf(x.x) + fabsf(x.y)) + (fabsf(x.z) + fabsf(x.w));
  }
  return n1;
}

template <int MODE>
struct LaneState;

template <>
struct LaneState<kModeDraft> : DraftLane {};

template <>
struct LaneState<kModeCstar> {
  double s;
  __device__ void init() { s = 0.0; }
};

template <>
struct LaneState<kModeResidual> {
  CandState cand;   // blocks of max(0, p^t - p^d)
  CandState candf;  // blocks of p^t
  float wpos;
  u32x4 words;
  __device__ void init() {
    cand.init();
    candf.init();
    wpos = 0.f;
  }
};

// Per-tile epilogue: the lane holds the draft logits z[j] = U + B of tokens
// vb + j (j < 16) of one row (block t = its tile) and, in the verify modes, the
// target logits tv[j]; entries at or beyond V hold -inf.  Exponentials are
// taken in base 2 with the scaling folded into one fma.
// dz bounds the binary32 contraction error of every logit of the tile
// (kContractErr ||W1[x]||_1 max|W2| over the tile).
// The draft passes the backbone logits u and the bias b separately (its
// log-sums are rounded relative to the block maximum only, see
// draft_block_epilogue); z = u + b for the other modes.
template <int MODE>
__device__ __forceinline__ void epilogue(LaneState<MODE>& st, const float* z, const float* tv,
                                         const RowCtx& rc, int t, bool first, uint64_t seed,
                                         float dz, const float* u = nullptr) {
  if constexpr (MODE == kModeDraft) {
    draft_block_epilogue(st, u, z, rc.r, rc.k, t, first, seed, dz);
  } else if constexpr (MODE == kModeCstar) {
    float e[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      e[j] = __builtin_amdgcn_exp2f(fminf(fmaf(z[j], kLog2e, -rc.ld2), fmaf(tv[j], kLog2e, -rc.lt2)));
    st.s += (double)sum16(e);
  } else {
    float w = 0.f, p = 0.f, q = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float pd = __builtin_amdgcn_exp2f(fmaf(z[j], kLog2e, -rc.ld2));
      const float pt = __builtin_amdgcn_exp2f(fmaf(tv[j], kLog2e, -rc.lt2));
      w += fmaxf(pt - pd, 0.f);
      p += pt + pd;
      q += pt;
    }
    const float W = sum_halves(w);
    const float P = sum_halves(p);
    const float Q = sum_halves(q);
    if (first || (t & 3) == 0) st.words = noise_block(seed, kStreamResidual, rc.r, rc.k, (uint32_t)t >> 2);
    const float g = gumbel_f32(word_of(st.words, t & 3));
    constexpr float kG = 0x1p-13f;  // Gumbel and log2 rounding
    st.wpos += W;
    const float err = (rc.eps + dz) * P;
    if (W + err > 0.f) {
      const float hi = fmaf(__builtin_amdgcn_logf(W + err), kLn2, g) + kG;
      const float lo = (W > err) ? fmaf(__builtin_amdgcn_logf(W - err), kLn2, g) - kG : -INFINITY;
      st.cand.add(lo, hi, t);
    }
    if (Q > 0.f) {
      const float lq = fmaf(__builtin_amdgcn_logf(Q), kLn2, g);
      const float dq = rc.eps + kG;
      st.candf.add(lq - dq, lq + dq, t);
    }
  }
}

// Partial record of the split for the lane's row, written by the lower half of
// the wave (both halves hold the same row; the c* sums are per half).
template <int MODE>
__device__ __forceinline__ void finish(const LaneState<MODE>& st, const RowCtx& rc, int row,
                                       int split, const BiasPassArgs& a, bool writer) {
  const int64_t o = (int64_t)row * a.rec_stride + split;
  if constexpr (MODE == kModeDraft) {
    if (writer && rc.active) {
      a.pm[o] = st.M;
      a.ps[o] = st.S;
      st.cand.store(a.cand, o);
    }
  } else if constexpr (MODE == kModeCstar) {
    const double s = st.s + xor32(st.s);
    if (writer && rc.active) a.ps[o] = s;
  } else {
    if (writer && rc.active) {
      st.cand.store(a.cand, o);
      st.candf.store(a.cand_f, o);
      a.wpos[o] = st.wpos;
    }
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// One pipeline stage = 2 tiles (64 tokens).  Every wave prefetches D stages
// (2 measured best) ahead into registers: its 1/8 share of the stage's packed W2 tiles (4 x 16 B
// per lane) and the 128-byte segments of its own 32 rows of U (and T), 8 rows
// x 128 B per load instruction.  At its turn a stage is written to LDS: the W2
// tiles to a double-buffered workgroup area, the row segments to the wave's
// own area (xor-swizzled 16-byte slots); one barrier per stage publishes the
// W2 tiles.  VEC: rows 16-byte aligned (vector loads), else scalar loads.
// One (split, row block) of a pass with `nsplit` splits.
// ZOUT (draft only): also store every logit z = U + B of the pass to a.zout.
template <int MODE, int D, bool VEC, bool ZOUT>
__device__ void bias_body(const BiasPassArgs& a, int split, int nsplit, int row_block,
                          int active_rows, int kpos) {
  constexpr bool kNeedT = MODE != kModeDraft;
  constexpr int ST = 2;
  constexpr int SEG = ST * 64;     // bytes of one row per stage
  constexpr int NSEG = SEG / 16;   // 16-byte segments of one row per stage
  constexpr int kABytes = ST * kTileBytesA;
  constexpr int NR = kNeedT ? 2 : 1;
  // the draft has the registers to batch the A-fragment reads of a tile
  constexpr bool kBatchA = !kNeedT;
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kABytes];
  __shared__ __attribute__((aligned(16))) uint8_t sR[kWaves][NR][32 * SEG];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;
  const int row0 = row_block * kRowsPerBlock;
  if (row0 >= active_rows) return;
  const int t_begin = split_tile(split, nsplit, a.ntiles, ST);
  const int t_end = split_tile(split + 1, nsplit, a.ntiles, ST);
  const int c_begin = t_begin / ST;
  const int c_end = (t_end + ST - 1) / ST;

  const int row = row0 + wave * 32 + n;
  // a wave without rows (a partial row block) stages its share of each stage
  // and meets the barriers but computes nothing: its matrix-core chains would
  // take the matrix unit from the live wave on the same SIMD
  const bool wave_live = row0 + wave * 32 < active_rows;
  // the draft's B operands come ready-made from the previous position's select
  // (a.bop), except at the first position
  const bool bop_ready = MODE == kModeDraft && a.bop != nullptr;
  const RowCtx rc = row_ctx(a, row, active_rows, true, kpos, !bop_ready);
  LaneState<MODE> st;
  st.init();

  // Row loads: instruction i covers rows 8i .. 8i+7 of the wave; lane -> row
  // 8i + lane/8, segment lane%8 of the stage's 128 bytes.
  const uint16_t* urow = rc.active ? reinterpret_cast<const uint16_t*>(rc.urow) : nullptr;
  const uint16_t* trow = (rc.active && kNeedT) ? reinterpret_cast<const uint16_t*>(rc.trow) : nullptr;
  const int lseg = lane & 7;
  const uint16_t* ld_u[4];
  const uint16_t* ld_t[4];
  int ld_slot[4];  // LDS byte offset of the lane's segment in the wave's area
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int nn = 8 * i + (lane >> 3);
    ld_u[i] = reinterpret_cast<const uint16_t*>(__shfl((unsigned long long)(uintptr_t)urow, nn, 64));
    ld_t[i] = reinterpret_cast<const uint16_t*>(__shfl((unsigned long long)(uintptr_t)trow, nn, 64));
    ld_slot[i] = (nn * NSEG + (lseg ^ seg_swz<NSEG>(nn))) * 16;
  }
  const u32x4* W2q = reinterpret_cast<const u32x4*>(a.W2p);

  // Stages c >= c_end are padding (the loop runs whole groups of D stages so
  // that every stage issues the same loads): their loads read one cached
  // 16-byte line and nothing they bring is used.
  u32x4 ra[D][4], ru[D][4], rt[D][kNeedT ? 4 : 1];
  auto row_seg = [&](const uint16_t* r, int v, bool live) -> u32x4 {
    if constexpr (VEC) {
      const bool in = live && r != nullptr && v + 8 <= a.V;
      const void* src = in ? static_cast<const void*>(r + v) : static_cast<const void*>(kNegInfBf16x8);
      if constexpr (kNeedT) return gload16_nt(src);
      else return gload16(src);
    } else {
      return live ? chunk_load(r, v, a.V) : gload16(kNegInfBf16x8);
    }
  };
  auto load_stage = [&](int d, int c) {
    const bool live = c < c_end;
    const int t0 = c * ST;
    // W2 chunks are loaded on every stage, tiles past the split clamped to its
    // last tile (already in L2; the copy is never read).  A load that depended
    // on `live` would let the compiler fold a constant source and drop loads on
    // that path, which breaks its exact count of loads in flight (it then
    // over-waits).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = wave * 256 + i * 64 + lane;  // 16-byte chunk of the stage's W2 tiles
      const int tt = min(t0 + (q >> 10), t_end - 1);
      ra[d][i] = gload16(W2q + (int64_t)tt * 1024 + (q & 1023));
    }
    const int v = t0 * kTile + lseg * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ru[d][i] = row_seg(ld_u[i], v, live);
      if constexpr (kNeedT) rt[d][i] = row_seg(ld_t[i], v, live);
    }
  };
  auto store_stage = [&](int d, int c) {
    uint8_t* da = sA[c & 1];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(da + (wave * 256 + i * 64 + lane) * 16) = ra[d][i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&sR[wave][0][ld_slot[i]]) = ru[d][i];
      if constexpr (kNeedT) *reinterpret_cast<u32x4*>(&sR[wave][NR - 1][ld_slot[i]]) = rt[d][i];
    }
  };

  // Stage 0's loads, then the W1 gather (which waits on the previous token),
  // then the later stages; one explicit wait leaves exactly the later stages in
  // flight.  The compiler sees the wait, so the loop needs no further wait for
  // the W1 rows (otherwise every tile drains the prefetch).
  load_stage(0, c_begin);
  bf16x8 bop[kSteps];
  if (bop_ready) {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.bop) + bop_chunk(row, 0, h);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const u32x4 v = src[s * 64];
      bop[s] = as_bf16x8(rc.active ? v : (u32x4){0u, 0u, 0u, 0u});
    }
  } else {
    const u32x4* w1 = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint16_t*>(a.W1) + (int64_t)rc.prev * kRank + 128 * h);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) bop[s] = as_bf16x8(rc.active ? w1[s] : (u32x4){0u, 0u, 0u, 0u});
  }
#pragma unroll
  for (int d = 1; d < D; ++d) load_stage(d, c_begin + d);
  {
    constexpr int kLoadsPerStage = 4 * (kNeedT ? 3 : 2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerStage * (D - 1)));
  }
  // ||W1[x]||_1 of the lane's row (each half of the wave holds half the rank)
  float n1 = 0.f;
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const u32x4 v = __builtin_bit_cast(u32x4, bop[s]);
    n1 += (fabsf(bf16_lo(v.x)) + fabsf(bf16_hi(v.x))) + (fabsf(bf16_lo(v.y)) + fabsf(bf16_hi(v.y))) +
          (fabsf(bf16_lo(v.z)) + fabsf(bf16_hi(v.z))) + (fabsf(bf16_lo(v.w)) + fabsf(bf16_hi(v.w)));
  }
  const float kz = kContractErr * sum_halves(n1);
  const float* tmax = w2_tile_absmax(a.W2p, true, a.ntiles);
  float* zrow = nullptr;
  if constexpr (ZOUT)
    if (rc.active) zrow = a.zout + ((int64_t)rc.r * a.gamma + (rc.k - 1)) * (int64_t)a.V;

  const int sw = seg_swz<NSEG>(n);
  const int c_stop = c_begin + (c_end - c_begin + D - 1) / D * D;
  for (int cb = c_begin; cb < c_stop; cb += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int c = cb + d;
      store_stage(d, c);
      load_stage(d, c + D);
      stage_barrier();  // stage c's W2 tiles visible to every wave
      if (c < c_end && wave_live) {
        const uint8_t* ra_lds = sA[c & 1];
        const uint8_t* ru_lds = &sR[wave][0][n * SEG];
        const uint8_t* rt_lds = &sR[wave][NR - 1][n * SEG];
#pragma unroll
        for (int tau = 0; tau < ST; ++tau) {
          const int t = c * ST + tau;
          if (t < t_end) {
            // draft and residual: the chain accumulates B from zero (its error
            // then scales with sum |W1 W2| only, which the brackets use) and the
            // backbone logits are added after it; c* (no bracket) seeds the
            // accumulator with them, so that the chain yields z = U + B
            const int s0 = 4 * tau + 2 * h;
            const float dz = kz * tile_absmax(tmax, t);
            f32x16 acc;
            if constexpr (MODE == kModeCstar) {
              float zu[16];
              decode16(*reinterpret_cast<const u32x4*>(ru_lds + ((s0 ^ sw) * 16)),
                       *reinterpret_cast<const u32x4*>(ru_lds + (((s0 + 1) ^ sw) * 16)), zu);
#pragma unroll
              for (int j = 0; j < 16; ++j) acc[j] = zu[j];
            } else {
#pragma unroll
              for (int j = 0; j < 16; ++j) acc[j] = 0.f;
            }
            const u32x4* At = reinterpret_cast<const u32x4*>(ra_lds + tau * kTileBytesA) + lane;
            if constexpr (kBatchA) {
              // all 16 A fragments in flight before the chain starts (one LDS
              // latency per tile instead of one per MFMA pair)
              u32x4 av[kSteps];
#pragma unroll
              for (int s = 0; s < kSteps; ++s) av[s] = At[s * 64];
              __builtin_amdgcn_sched_barrier(0);
#pragma unroll
              for (int s = 0; s < kSteps; ++s)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[s]), bop[s], acc, 0, 0, 0);
            } else {
#pragma unroll
              for (int s = 0; s < kSteps; ++s)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(At[s * 64]), bop[s], acc, 0, 0, 0);
            }
            float z[16], zu[16];
            if constexpr (MODE == kModeCstar) {
#pragma unroll
              for (int j = 0; j < 16; ++j) z[j] = acc[j];
            } else {
              decode16(*reinterpret_cast<const u32x4*>(ru_lds + ((s0 ^ sw) * 16)),
                       *reinterpret_cast<const u32x4*>(ru_lds + (((s0 + 1) ^ sw) * 16)), zu);
#pragma unroll
              for (int j = 0; j < 16; ++j) z[j] = (MODE == kModeDraft) ? acc[j] : zu[j] + acc[j];
            }
            if constexpr (ZOUT) {
              const int vb = t * kTile + 16 * h;
              if (zrow)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                  if (vb + j < a.V) zrow[vb + j] = zu[j] + z[j];
            }
            float tv[16];
            if constexpr (kNeedT)
              decode16(*reinterpret_cast<const u32x4*>(rt_lds + ((s0 ^ sw) * 16)),
                       *reinterpret_cast<const u32x4*>(rt_lds + (((s0 + 1) ^ sw) * 16)), tv);
            epilogue<MODE>(st, z, tv, rc, t, t == t_begin, a.seed, dz, zu);
          }
        }
      }
    }
  }
  finish<MODE>(st, rc, row, split, a, h == 0);
}

// The workgroup's (split, split count, row block).  Static passes: the grid
// is (splits, row blocks).  With `dyn` the launched workgroups are spread over
// the row blocks that hold active rows (active_split_count).
struct PassWork {
  int split, nsplit, row_block;
};

__device__ __forceinline__ PassWork pass_work(const BiasPassArgs& a, int active_rows) {
  if (!a.dyn) return {(int)blockIdx.x, a.nsplit, (int)blockIdx.y};
  const int grid = (int)(gridDim.x * gridDim.y);
  const int id = (int)(blockIdx.x + gridDim.x * blockIdx.y);
  const int ns = active_split_count(grid, active_rows, a.rec_stride);
  return {id % ns, ns, id / ns};
}

template <int MODE, int D, bool VEC, bool ZOUT = false>
__global__ __launch_bounds__(kThreads) void k_bias_bf16(const BiasPassArgs a) {
  const int active_rows = a.row_count ? min(*a.row_count, a.nrows) : a.nrows;
  const PassWork w = pass_work(a, active_rows);
  bias_body<MODE, D, VEC, ZOUT>(a, w.split, w.nsplit, w.row_block, active_rows, a.k);
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
  const PassWork work = pass_work(a, active_rows);
  const int row0 = work.row_block * kRowsPerBlock;
  if (row0 >= active_rows) return;
  const int split = work.split;
  const int t_begin = split_tile(split, work.nsplit, a.ntiles, a.tiles_per_stage);
  const int t_end = split_tile(split + 1, work.nsplit, a.ntiles, a.tiles_per_stage);
  const f32x4* W2T = reinterpret_cast<const f32x4*>(a.W2p);
  const float* tmax = w2_tile_absmax(a.W2p, false, a.ntiles);
  constexpr bool kNeedT = MODE != kModeDraft;

  if (active_rows - row0 <= 32) {
    // At most one wave's rows: the 8 waves share them and split the rank
    // instead, wave w summing ranks [32w, 32w + 32); wave 0 adds the eight
    // partial sums in a fixed order and runs the epilogue.  Each tile's slice
    // of the transposed W2 (32 tokens x 256, 32 KB) is staged in LDS with one
    // coalesced load per thread quad, the next tile's slice in flight meanwhile.
    __shared__ float part[kWaves][16][64];
    __shared__ f32x4 sW[2][kTile * (kRank / 4)];
    const int row = row0 + n;
    const RowCtx rc = row_ctx(a, row, active_rows, false, a.k);
    LaneState<MODE> st;
    st.init();
    const f32x4* w1 = reinterpret_cast<const f32x4*>(
        reinterpret_cast<const float*>(a.W1) + (int64_t)rc.prev * kRank);
    const float* ur = reinterpret_cast<const float*>(rc.urow);
    const float* tr = reinterpret_cast<const float*>(rc.trow);
    const float kz = kContractErr * (rc.active ? w1_norm1(w1) : 0.f);
    float* zrow = (MODE == kModeDraft && a.zout && rc.active)
                      ? a.zout + ((int64_t)rc.r * a.gamma + (rc.k - 1)) * (int64_t)a.V
                      : nullptr;
    f32x4 xw[8];  // this wave's 32 ranks of the row's W1 operand
#pragma unroll
    for (int q = 0; q < 8; ++q) xw[q] = rc.active ? w1[8 * wave + q] : (f32x4){0.f, 0.f, 0.f, 0.f};
    constexpr int kSlice = kTile * (kRank / 4);        // 2048 f32x4 per tile
    constexpr int kPer = kSlice / kThreads;             // 4 per thread
    f32x4 pre[kPer];
    auto load_slice = [&](int t) {
#pragma unroll
      for (int q = 0; q < kPer; ++q) pre[q] = W2T[(int64_t)t * kSlice + tid + q * kThreads];
    };
    if (t_begin < t_end) load_slice(t_begin);
    for (int t = t_begin; t < t_end; ++t) {
      const int buf = (t - t_begin) & 1;
#pragma unroll
      for (int q = 0; q < kPer; ++q) sW[buf][tid + q * kThreads] = pre[q];
      if (t + 1 < t_end) load_slice(t + 1);
      stage_barrier();  // the slice is visible; the loads of the next stay in flight
      const int vb = t * kTile + 16 * h;
      float acc[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = 0.f;
      if (rc.active) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const f32x4 x = xw[q];
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const f32x4 y = sW[buf][(16 * h + j) * (kRank / 4) + 8 * wave + q];
            acc[j] = fmaf(x.x, y.x, acc[j]);
            acc[j] = fmaf(x.y, y.y, acc[j]);
            acc[j] = fmaf(x.z, y.z, acc[j]);
            acc[j] = fmaf(x.w, y.w, acc[j]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) part[wave][j][lane] = acc[j];
      stage_barrier();  // LDS only: the next slice's loads stay in flight
      if (wave == 0) {
        float z[16], zu[16], tv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          float b = part[0][j][lane];
          for (int w = 1; w < kWaves; ++w) b += part[w][j][lane];
          zu[j] = (rc.active && vb + j < a.V) ? ur[vb + j] : -INFINITY;
          z[j] = (MODE == kModeDraft) ? b : zu[j] + b;  // the draft takes u and b apart
          tv[j] = (kNeedT && rc.active && vb + j < a.V) ? tr[vb + j] : -INFINITY;
          if (zrow && vb + j < a.V) zrow[vb + j] = zu[j] + b;
        }
        epilogue<MODE>(st, z, tv, rc, t, t == t_begin, a.seed, kz * tile_absmax(tmax, t), zu);
      }
      stage_barrier();
    }
    if (wave == 0) finish<MODE>(st, rc, row, split, a, h == 0);
    return;
  }

  const int row = row0 + wave * 32 + n;
  const RowCtx rc = row_ctx(a, row, active_rows, false, a.k);
  LaneState<MODE> st;
  st.init();
  if (rc.active) {
    const f32x4* w1 = reinterpret_cast<const f32x4*>(
        reinterpret_cast<const float*>(a.W1) + (int64_t)rc.prev * kRank);
    const float* ur = reinterpret_cast<const float*>(rc.urow);
    const float* tr = reinterpret_cast<const float*>(rc.trow);
    const float kz = kContractErr * w1_norm1(w1);
    float* zrow = (MODE == kModeDraft && a.zout)
                      ? a.zout + ((int64_t)rc.r * a.gamma + (rc.k - 1)) * (int64_t)a.V
                      : nullptr;
    for (int t = t_begin; t < t_end; ++t) {
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
      float z[16], zu[16], tv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        zu[j] = (vb + j < a.V) ? ur[vb + j] : -INFINITY;
        z[j] = (MODE == kModeDraft) ? acc[j] : zu[j] + acc[j];  // the draft takes u and b apart
        tv[j] = (kNeedT && vb + j < a.V) ? tr[vb + j] : -INFINITY;
        if (zrow && vb + j < a.V) zrow[vb + j] = zu[j] + acc[j];
      }
      epilogue<MODE>(st, z, tv, rc, t, t == t_begin, a.seed, kz * tile_absmax(tmax, t), zu);
    }
  }
  finish<MODE>(st, rc, row, split, a, h == 0);
}

// Draft and residual passes for at most 32 rows (one 32-row group, bf16):
// with a single row group nothing is worth sharing between waves, so every
// wave streams its own contiguous quarter of the workgroup's tiles with no LDS
// staging and no barrier: the A operands (packed W2 tile) and the lane's 16
// backbone logits (and target logits) are loaded straight into registers, one
// tile ahead, and each W2 tile crosses the fabric once per launch.  Workgroup
// = split (tile-granular); the four waves' states of each row are merged
// through LDS at the end.
template <int MODE, bool VEC, bool ZOUT>
__global__ __launch_bounds__(256) void k_bias_small(const BiasPassArgs a) {
  constexpr int kW = 4;
  constexpr bool kNeedT = MODE != kModeDraft;
  static_assert(MODE == kModeDraft || MODE == kModeResidual, "draft or residual");
  static_assert(!ZOUT || MODE == kModeDraft, "logits out in the draft only");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;
  const int active_rows = a.row_count ? min(*a.row_count, a.nrows) : a.nrows;
  if (active_rows <= 0) return;
  const int split = blockIdx.x;
  const int t0 = split_tile(split, a.nsplit, a.ntiles, 1);
  const int t1 = split_tile(split + 1, a.nsplit, a.ntiles, 1);
  const int per = (t1 - t0 + kW - 1) / kW;
  const int tb = min(t1, t0 + wave * per);
  const int te = min(t1, tb + per);
  const bool bop_ready = MODE == kModeDraft && a.bop != nullptr;
  const RowCtx rc = row_ctx(a, n, active_rows, true, a.k, !bop_ready);
  LaneState<MODE> st;
  st.init();

  bf16x8 bop[kSteps];
  if (bop_ready) {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.bop) + bop_chunk(n, 0, h);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const u32x4 v = src[s * 64];
      bop[s] = as_bf16x8(rc.active ? v : (u32x4){0u, 0u, 0u, 0u});
    }
  } else {
    const u32x4* w1 = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint16_t*>(a.W1) + (int64_t)rc.prev * kRank + 128 * h);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) bop[s] = as_bf16x8(rc.active ? w1[s] : (u32x4){0u, 0u, 0u, 0u});
  }
  float n1 = 0.f;
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const u32x4 v = __builtin_bit_cast(u32x4, bop[s]);
    n1 += (fabsf(bf16_lo(v.x)) + fabsf(bf16_hi(v.x))) + (fabsf(bf16_lo(v.y)) + fabsf(bf16_hi(v.y))) +
          (fabsf(bf16_lo(v.z)) + fabsf(bf16_hi(v.z))) + (fabsf(bf16_lo(v.w)) + fabsf(bf16_hi(v.w)));
  }
  const float kz = kContractErr * sum_halves(n1);
  const float* tmax = w2_tile_absmax(a.W2p, true, a.ntiles);
  const u32x4* W2q = reinterpret_cast<const u32x4*>(a.W2p);
  const uint16_t* urow = rc.active ? reinterpret_cast<const uint16_t*>(rc.urow) : nullptr;
  const uint16_t* trow = (kNeedT && rc.active) ? reinterpret_cast<const uint16_t*>(rc.trow) : nullptr;
  float* zrow = nullptr;
  if constexpr (ZOUT)
    if (rc.active) zrow = a.zout + ((int64_t)rc.r * a.gamma + (rc.k - 1)) * (int64_t)a.V;

  // the lane's 16 logits [v, v + 16) of a row (-inf beyond V and for a null row)
  auto row16 = [&](const uint16_t* row, int v, u32x4& lo, u32x4& hi) {
    if (VEC && row != nullptr && v + 16 <= a.V) {
      if constexpr (kNeedT) {
        lo = gload16_nt(row + v);
        hi = gload16_nt(row + v + 8);
      } else {
        lo = gload16(row + v);
        hi = gload16(row + v + 8);
      }
    } else {
      lo = chunk_load(row, v, a.V);
      hi = chunk_load(row, v + 8, a.V);
    }
  };
  // tile loads: 16 A fragments and the lane's logits (tiles past the wave's
  // range repeat its last tile and are never used)
  struct Tile {
    u32x4 A[kSteps];
    u32x4 ulo, uhi, tlo, thi;
  };
  auto load_tile = [&](int t, Tile& x) {
    const int tt = min(t, max(te - 1, tb));
#pragma unroll
    for (int s = 0; s < kSteps; ++s) x.A[s] = gload16(W2q + (int64_t)tt * 1024 + s * 64 + lane);
    const int v = tt * kTile + 16 * h;
    row16(urow, v, x.ulo, x.uhi);
    if constexpr (kNeedT) row16(trow, v, x.tlo, x.thi);
  };
  Tile cur;
  if (tb < te) load_tile(tb, cur);
  for (int t = tb; t < te; ++t) {
    Tile nxt;
    load_tile(t + 1, nxt);  // one tile ahead
    f32x16 acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur.A[s]), bop[s], acc, 0, 0, 0);
    float z[16], zu[16], tv[16];
    decode16(cur.ulo, cur.uhi, zu);
    // the draft passes the bias and the backbone logits apart, the residual z
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = (MODE == kModeDraft) ? acc[j] : zu[j] + acc[j];
    if constexpr (kNeedT) decode16(cur.tlo, cur.thi, tv);
    if constexpr (ZOUT) {
      const int vb = t * kTile + 16 * h;
      if (zrow)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (vb + j < a.V) zrow[vb + j] = zu[j] + z[j];
    }
    epilogue<MODE>(st, z, tv, rc, t, t == tb, a.seed, kz * tile_absmax(tmax, t), zu);
    cur = nxt;
  }

  // merge the four waves' states of each row (disjoint tile ranges)
  if constexpr (MODE == kModeDraft) {
    __shared__ float sm[kW][32], slo[kW][32], shi1[kW][32], shi2[kW][32];
    __shared__ double ss[kW][32];
    __shared__ int sb1[kW][32];
    if (h == 0) {
      sm[wave][n] = st.M;
      ss[wave][n] = st.S;
      slo[wave][n] = st.cand.lo;
      shi1[wave][n] = st.cand.hi1;
      shi2[wave][n] = st.cand.hi2;
      sb1[wave][n] = st.cand.b1;
    }
    __syncthreads();
    if (wave == 0) {
      for (int w = 1; w < kW; ++w) {
        lse_merge(st.M, st.S, sm[w][n], ss[w][n]);
        CandState o;
        o.lo = slo[w][n];
        o.hi1 = shi1[w][n];
        o.hi2 = shi2[w][n];
        o.b1 = sb1[w][n];
        st.cand.merge(o);
      }
      finish<MODE>(st, rc, n, split, a, h == 0);
    }
  } else {
    __shared__ CandState sc[kW][32], sf[kW][32];
    __shared__ float sw[kW][32];
    if (h == 0) {
      sc[wave][n] = st.cand;
      sf[wave][n] = st.candf;
      sw[wave][n] = st.wpos;
    }
    __syncthreads();
    if (wave == 0) {
      for (int w = 1; w < kW; ++w) {
        st.cand.merge(sc[w][n]);
        st.candf.merge(sf[w][n]);
        st.wpos += sw[w][n];
      }
      finish<MODE>(st, rc, n, split, a, h == 0);
    }
  }
}

}  // namespace

// Vocabulary splits: enough workgroups for one full round on MI355X (256 CUs,
// one 8-wave workgroup each), never more splits than pipeline stages (2 tiles
// in the bf16 passes; the binary32 pass works tile by tile).
BiasGeometry bias_geometry(int mode, bool bf16, int nrows, int V) {
  constexpr int kSlots = 256;
  BiasGeometry g;
  g.rows_per_block = kRowsPerBlock;
  g.row_blocks = (nrows + kRowsPerBlock - 1) / kRowsPerBlock;
  g.tiles_per_stage = bf16 ? 2 : 1;
  const int ntiles = (V + kTile - 1) / kTile;
  const int nstages = (ntiles + g.tiles_per_stage - 1) / g.tiles_per_stage;
  g.nsplit = min(nstages, max(1, (kSlots + g.row_blocks - 1) / g.row_blocks));
  return g;
}

int small_pass_splits(int nrows, int V) {
  const int ntiles = (V + kTile - 1) / kTile;
  return nrows <= 32 ? min(ntiles, 256) : 0;
}

hipError_t launch_bias_pass(int mode, bool bf16, const BiasPassArgs& a, hipStream_t stream) {
  TimingScope timing(mode == kModeDraft ? "draft_bias" : (mode == kModeCstar ? "cstar_bias" : "residual_bias"), stream);
  const dim3 grid(a.nsplit, (a.nrows + kRowsPerBlock - 1) / kRowsPerBlock);
  const dim3 block(kThreads);
  if (bf16 && mode != kModeCstar && a.tiles_per_stage == 1) {  // at most 32 rows
    if (a.nrows > 32) return hipErrorInvalidValue;
    const dim3 g(a.nsplit), b(256);
    if (mode == kModeResidual) {
      if (a.vec_ok) hipLaunchKernelGGL((k_bias_small<kModeResidual, true, false>), g, b, 0, stream, a);
      else hipLaunchKernelGGL((k_bias_small<kModeResidual, false, false>), g, b, 0, stream, a);
    } else if (a.vec_ok && a.zout) {
      hipLaunchKernelGGL((k_bias_small<kModeDraft, true, true>), g, b, 0, stream, a);
    } else if (a.vec_ok) {
      hipLaunchKernelGGL((k_bias_small<kModeDraft, true, false>), g, b, 0, stream, a);
    } else if (a.zout) {
      hipLaunchKernelGGL((k_bias_small<kModeDraft, false, true>), g, b, 0, stream, a);
    } else {
      hipLaunchKernelGGL((k_bias_small<kModeDraft, false, false>), g, b, 0, stream, a);
    }
  } else if (bf16 && mode == kModeDraft && a.zout) {
    if (a.vec_ok) hipLaunchKernelGGL((k_bias_bf16<kModeDraft, 2, true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k_bias_bf16<kModeDraft, 2, false, true>), grid, block, 0, stream, a);
  } else if (bf16 && a.vec_ok) {
    if (mode == kModeDraft) hipLaunchKernelGGL((k_bias_bf16<kModeDraft, 2, true>), grid, block, 0, stream, a);
    else if (mode == kModeCstar) hipLaunchKernelGGL((k_bias_bf16<kModeCstar, 2, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k_bias_bf16<kModeResidual, 2, true>), grid, block, 0, stream, a);
  } else if (bf16) {
    if (mode == kModeDraft) hipLaunchKernelGGL((k_bias_bf16<kModeDraft, 2, false>), grid, block, 0, stream, a);
    else if (mode == kModeCstar) hipLaunchKernelGGL((k_bias_bf16<kModeCstar, 2, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k_bias_bf16<kModeResidual, 2, false>), grid, block, 0, stream, a);
  } else {
    if (mode == kModeDraft) hipLaunchKernelGGL(k_bias_f32<kModeDraft>, grid, block, 0, stream, a);
    else if (mode == kModeCstar) hipLaunchKernelGGL(k_bias_f32<kModeCstar>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(k_bias_f32<kModeResidual>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dspark
