// verify_aux.hip -- the verification steps that need no Markov-head bias:
//   build_rows : (request, position) rows to verify, k <= l_r (with per-request
//                lengths; when every position is verified the target pass
//                writes the identity row map)
//   target_lse : log-sum-exp of every verified target row (split vocabulary)
//   decide     : acceptance test of each drafted token, first rejection,
//                residual / bonus work lists (standard speculative rejection
//                sampling; notes page 배경, summary page 요약)
//   bonus      : first level of the two-level Gumbel-max draw over T[r, l_r]
//                when every verified token is accepted (bonus token from p^t_{l_r+1});
//                its first split's workgroups also sum c* per (request, position)
#include "device_common.h"
#include "kernels.h"

namespace dspark {

namespace {

__device__ __forceinline__ void load8(const uint16_t* row, int v, int vend, bool vec_ok, float* out) {
  if (vec_ok && v + 8 <= vend) {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + v));
    out[0] = bf16_lo(a.x); out[1] = bf16_hi(a.x);
    out[2] = bf16_lo(a.y); out[3] = bf16_hi(a.y);
    out[4] = bf16_lo(a.z); out[5] = bf16_hi(a.z);
    out[6] = bf16_lo(a.w); out[7] = bf16_hi(a.w);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = (v + i < vend) ? bf16_at(row, v + i) : -INFINITY;
  }
}

__device__ __forceinline__ void load8(const float* row, int v, int vend, bool vec_ok, float* out) {
  if (vec_ok && v + 8 <= vend) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + v));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + v) + 1);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = (v + i < vend) ? row[v + i] : -INFINITY;
  }
}

// Block-wide (256 threads) merge of (m, s) into thread 0.
__device__ __forceinline__ void block_lse(float& m, double& s) {
  __shared__ float sm[4];
  __shared__ double ss[4];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const double s2 = __shfl_xor(s, off, 64);
    lse_merge(m, s, m2, s2);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) lse_merge(m, s, sm[w], ss[w]);
  }
  __syncthreads();
}

__global__ __launch_bounds__(1024) void k_build_rows(int R, int gamma, const int32_t* lengths,
                                                     VerifyWs w) {
  __shared__ int scan[1024];
  __shared__ int carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < R; base += 1024) {
    const int r = base + tid;
    int L = 0;
    if (r < R) L = lengths ? min(max(lengths[r], 0), gamma) : gamma;
    scan[tid] = L;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int excl = carry + scan[tid] - L;
    if (r < R) {
      w.req_off[r] = excl;
      w.req_len[r] = L;
      w.req_mode[r] = 0;
      w.req_slot[r] = 0;
      for (int k = 1; k <= L; ++k) w.row_ids[excl + k - 1] = r * gamma + (k - 1);
    }
    __syncthreads();
    if (tid == 1023) carry += scan[1023];
    __syncthreads();
  }
  if (tid == 0) {
    w.counts[0] = carry;
    w.counts[1] = 0;
    w.counts[2] = 0;
    w.counts[3] = 0;
  }
}

// Workgroup id = verified row * splits + split, the split count following the
// device row count (lse_split_count; records at stride ns_t).
template <typename E>
__global__ __launch_bounds__(256) void k_target_lse(int gamma, int V, const E* T, VerifyWs w) {
  const int nrows = (int)gridDim.x;  // every position
  const bool all = w.all_rows != 0;
  if (all && blockIdx.y == 0 && threadIdx.x == 0) {
    // every position verified: the row map is the identity, written here in
    // place of a row-building pass (later kernels read it; this one does not)
    const int x = (int)blockIdx.x;
    w.row_ids[x] = x;
    if (x < nrows / gamma) {
      w.req_off[x] = x * gamma;
      w.req_len[x] = gamma;
      w.req_mode[x] = 0;
      w.req_slot[x] = 0;
    }
    if (x == 0) {
      w.counts[0] = nrows;
      w.counts[1] = 0;
      w.counts[2] = 0;
      w.counts[3] = 0;
    }
  }
  const int active = all ? nrows : min(w.counts[0], nrows);
  int chunk;
  const int ns = lse_split_count(active, w.grid_t, V, &chunk);
  const int wg = (int)(blockIdx.x + gridDim.x * blockIdx.y);
  const int i = wg / ns;
  if (i >= active) return;
  const int split = wg - i * ns;
  const int id = all ? i : w.row_ids[i];
  const int r = id / gamma;
  const int k = id - r * gamma + 1;
  const E* row = T + ((int64_t)r * (gamma + 1) + (k - 1)) * (int64_t)V;
  const int v0 = split * chunk;
  const int v1 = min(V, v0 + chunk);
  const bool vec_ok = w.vec_ok != 0;
  // Running max m and s = sum 2^(x L - K) against an integer reference
  // K = ceil(fl(m L)) (L = log2 e in binary32).  Each exponent is one fma,
  // fma(x, L, -K), rounded relative to |x L - K| only; a rise of K rescales s
  // by an exact power of two (the wave meets a new maximum in some lane at
  // almost every step, so this branch must stay cheap).  At the end s is
  // brought to sum exp(x - m) by the factor 2^(K - m L), in binary64 with the
  // same L, so that an element's residual scaling error is |x - m| times the
  // error of L only.
  float m = -INFINITY, kf = 0.f;
  double s = 0.0;
  for (int v = v0; v < v1; v += 16 * 256) {
    float x[16];
    load_slice16(row, v, (int)threadIdx.x, v1, vec_ok, x);
    float mt = x[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mt = fmaxf(mt, x[j]);
    if (mt > m) {
      const float kn = ceilf(mt * kLog2e);
      if (m == -INFINITY) {
        kf = kn;
      } else if (kn > kf) {
        s = ldexp(s, (int)fmax((double)kf - (double)kn, -2000.0));
        kf = kn;
      }
      m = mt;
    }
    if (m != -INFINITY) {
      float e[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) e[j] = __builtin_amdgcn_exp2f(fmaf(x[j], kLog2e, -kf));
      const float a0 = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      const float a1 = ((e[8] + e[9]) + (e[10] + e[11])) + ((e[12] + e[13]) + (e[14] + e[15]));
      s += (double)(a0 + a1);
    }
  }
  if (m != -INFINITY) s *= exp2((double)kf - (double)m * (double)kLog2e);
  block_lse(m, s);
  if (threadIdx.x == 0) {
    const int64_t o = (int64_t)i * w.ns_t + split;  // ns_t: the record stride
    w.lt_m[o] = m;
    w.lt_s[o] = s;
  }
}

template <typename E>
__global__ __launch_bounds__(256) void k_decide(int R, int gamma, int V, uint64_t seed,
                                                const E* T, const int32_t* tokens,
                                                const double* logq, VerifyWs w,
                                                int32_t* n_accept, uint8_t* accept_mask,
                                                double* lse_t_out) {
  __shared__ double lse_k[64];
  __shared__ uint8_t ok_k[64];
  const int r = blockIdx.x;
  const int L = w.req_len[r];
  const int off = w.req_off[r];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // 0. what the acceptance test needs besides lse_t, fetched first so that the
  //    token -> T[x] round trip overlaps the merge of the lse partials:
  //    thread k - 1 holds position k's T[x], log q and ln u (gamma <= 64)
  double tx = 0.0, lq = 0.0, lnu = 0.0;
  const int kt = (int)threadIdx.x + 1;
  if (kt <= L) {
    const int64_t o = (int64_t)r * gamma + (kt - 1);
    const int x = min(max(tokens[o], 0), V - 1);
    tx = (double)elem_at(T, ((int64_t)r * (gamma + 1) + (kt - 1)) * (int64_t)V + x);
    lq = logq[o];
    lnu = log(uniform_f64(noise_block(seed, kStreamAccept, r, kt, 0).x));
  }
  // 1. lse of each verified target row: wave q merges the split partials of
  //    positions q + 1, q + 5, ... (no workgroup barrier per position)
  int chunk;
  const int ns = lse_split_count(min(w.counts[0], R * gamma), w.grid_t, V, &chunk);
  for (int k = wave + 1; k <= L; k += 4) {
    const int64_t base = (int64_t)(off + k - 1) * w.ns_t;
    float m = -INFINITY;
    double s = 0.0;
    for (int j = lane; j < ns; j += 64) lse_merge(m, s, w.lt_m[base + j], w.lt_s[base + j]);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float m2 = __shfl_xor(m, o, 64);
      const double s2 = __shfl_xor(s, o, 64);
      lse_merge(m, s, m2, s2);
    }
    if (lane == 0) lse_k[k - 1] = (double)m + log(s);
  }
  __syncthreads();
  for (int k = threadIdx.x + 1; k <= gamma + 1; k += 256) {
    const double v = (k <= L) ? lse_k[k - 1] : NAN;
    w.lse_t[(int64_t)r * (gamma + 1) + (k - 1)] = v;
    if (lse_t_out) lse_t_out[(int64_t)r * (gamma + 1) + (k - 1)] = v;
  }
  // 2. every verified position's test at once: accept x_k iff ln u < ln p^t(x_k) - ln p^d(x_k)
  if (kt <= L) ok_k[kt - 1] = lnu < (tx - lse_k[kt - 1]) - lq ? 1 : 0;
  __syncthreads();
  // 3. the first rejection ends the accepted prefix
  if (threadIdx.x == 0) {
    int n = L, kstar = 0;
    for (int k = 1; k <= gamma; ++k) {
      uint8_t mk = 255;
      if (k <= L && kstar == 0) {
        mk = ok_k[k - 1];
        if (!mk) {
          kstar = k;
          n = k - 1;
        }
      }
      if (accept_mask) accept_mask[(int64_t)r * gamma + (k - 1)] = mk;
    }
    n_accept[r] = n;
    if (kstar > 0) {
      const int slot = atomicAdd(&w.counts[1], 1);
      w.resid_ids[slot] = r * gamma + (kstar - 1);
      w.req_mode[r] = 1;
      w.req_slot[r] = slot;
    } else {
      const int slot = atomicAdd(&w.counts[2], 1);
      w.bonus_ids[slot] = r * (gamma + 1) + L;
      w.req_mode[r] = 2;
      w.req_slot[r] = slot;
    }
  }
}

// c* of request r's positions, one wave per position: the sum of the
// position's vocabulary splits (NaN beyond the request's verify length).  Run
// by the bonus pass, which follows the c* pass on the stream.
__device__ __forceinline__ void finalize_request(int r, int R, int gamma, const VerifyWs& w,
                                                 float* cstar) {
  const int lane = threadIdx.x & 63;
  // the c* pass's split count for this many verified rows (records at stride ns_c)
  const int ns = active_split_count(w.grid_c, min(w.counts[0], R * gamma), w.ns_c);
  const int L = w.req_len[r];
  for (int k = (int)(threadIdx.x >> 6) + 1; k <= gamma; k += 4) {
    const int64_t item = (int64_t)r * gamma + (k - 1);
    if (k > L) {
      if (lane == 0) cstar[item] = NAN;
      continue;
    }
    const int64_t base = (int64_t)(w.req_off[r] + k - 1) * w.ns_c;
    double s = 0.0;
    for (int j = lane; j < ns; j += 64) s += w.c_s[base + j];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) cstar[item] = (float)s;
  }
}

// Bonus draw, first level: per 32-token block of the target row T[r, l_r]
// (p^t_{l_r+1}), the block log-mass plus its Gumbel variate (stream 3), kept
// as split records for the binary64 select stage.  A quad of threads covers
// one block (8 tokens each).
// The workgroups of the first split also finalize c* of request blockIdx.x
// (the grid has one column per request).
template <typename E>
__global__ __launch_bounds__(256) void k_bonus(int gamma, int V, uint64_t seed, const E* T,
                                               VerifyWs w, float* cstar) {
  __shared__ float slo[4], shi1[4], shi2[4];
  __shared__ int sb1[4];
  const int i = blockIdx.x;
  if (blockIdx.y == 0) finalize_request(i, (int)gridDim.x, gamma, w, cstar);
  if (i >= w.counts[2]) return;
  const int id = w.bonus_ids[i];
  const int r = id / (gamma + 1);
  const int kb = id - r * (gamma + 1) + 1;
  const E* row = T + (int64_t)id * V;
  const int ntiles = (V + kTile - 1) / kTile;
  const int split = blockIdx.y;
  const int t0 = split_tile(split, w.ns_b, ntiles, 1);
  const int t1 = split_tile(split + 1, w.ns_b, ntiles, 1);
  const bool vec_ok = w.vec_ok != 0;
  CandState cs;
  cs.init();
  // Four 2048-token steps per iteration.  In every step the quad of a block
  // reduces its maximum and sum; thread q of the quad keeps step q's block, so
  // the per-block work (Philox block, Gumbel variate, logarithm, record) runs
  // on every lane once per four steps rather than on one lane in four per step.
  // The record keeps the largest bounds whatever the order the blocks come in
  // (an exact tie of upper bounds leaves hi2 = hi1, and every block of the
  // split is then rescored).
  const int vend = t1 * kTile;  // a multiple of 32: a quad is in or out as a whole
  const int q4 = (int)threadIdx.x & 3;
  for (int v0 = t0 * kTile + 8 * (int)threadIdx.x; v0 < vend; v0 += 4 * 8 * 256) {
    float km = -INFINITY, ks = 0.f;
    int kblk = -1;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + u * 8 * 256;
      if (v < vend) {
        float x[8];
        load8(row, v, V, vec_ok, x);
        float m = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        float s = 0.f;
        if (m > -INFINITY) {
          float e[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) e[j] = __builtin_amdgcn_exp2f((x[j] - m) * kLog2e);
          s = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
        }
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        if (q4 == u) {
          km = m;
          ks = s;
          kblk = v / kTile;
        }
      }
    }
    if (kblk >= 0 && km > -INFINITY) {
      const u32x4 words = noise_block(seed, kStreamBonus, r, kb, (uint32_t)kblk >> 2);
      const float sc = fmaf(__builtin_amdgcn_logf(ks), kLn2, km) + gumbel_f32(word_of(words, kblk & 3));
      const float d = fmaf(kScoreRel, fabsf(km), kScoreAbs);
      cs.add(sc - d, sc + d, kblk);
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    CandState o;
    o.lo = __shfl_xor(cs.lo, off, 64);
    o.hi1 = __shfl_xor(cs.hi1, off, 64);
    o.hi2 = __shfl_xor(cs.hi2, off, 64);
    o.b1 = __shfl_xor(cs.b1, off, 64);
    cs.merge(o);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    slo[wave] = cs.lo;
    shi1[wave] = cs.hi1;
    shi2[wave] = cs.hi2;
    sb1[wave] = cs.b1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int x = 1; x < 4; ++x) {
      CandState o;
      o.lo = slo[x];
      o.hi1 = shi1[x];
      o.hi2 = shi2[x];
      o.b1 = sb1[x];
      cs.merge(o);
    }
    cs.store(w.b_cand, (int64_t)i * w.ns_b + split);
  }
}

}  // namespace

hipError_t launch_build_rows(int R, int gamma, const int32_t* lengths, const VerifyWs& w,
                             hipStream_t stream) {
  TimingScope timing("build_rows", stream);
  hipLaunchKernelGGL(k_build_rows, dim3(1), dim3(1024), 0, stream, R, gamma, lengths, w);
  return hipGetLastError();
}

hipError_t launch_target_lse(bool bf16, int R, int gamma, int V, const void* T, const VerifyWs& w,
                             hipStream_t stream) {
  TimingScope timing("target_lse", stream);
  const dim3 grid(R * gamma, w.grid_t / (R * gamma));  // (positions, splits for every position)
  if (bf16)
    hipLaunchKernelGGL(k_target_lse<uint16_t>, grid, dim3(256), 0, stream, gamma, V,
                       (const uint16_t*)T, w);
  else
    hipLaunchKernelGGL(k_target_lse<float>, grid, dim3(256), 0, stream, gamma, V, (const float*)T, w);
  return hipGetLastError();
}

hipError_t launch_decide(bool bf16, int R, int gamma, int V, uint64_t seed, const void* T,
                         const int32_t* tokens, const double* logq, const VerifyWs& w,
                         int32_t* n_accept, uint8_t* accept_mask, double* lse_t_out,
                         hipStream_t stream) {
  TimingScope timing("decide", stream);
  if (bf16)
    hipLaunchKernelGGL(k_decide<uint16_t>, dim3(R), dim3(256), 0, stream, R, gamma, V, seed,
                       (const uint16_t*)T, tokens, logq, w, n_accept, accept_mask, lse_t_out);
  else
    hipLaunchKernelGGL(k_decide<float>, dim3(R), dim3(256), 0, stream, R, gamma, V, seed,
                       (const float*)T, tokens, logq, w, n_accept, accept_mask, lse_t_out);
  return hipGetLastError();
}

hipError_t launch_bonus(bool bf16, int R, int gamma, int V, uint64_t seed, const void* T,
                        const VerifyWs& w, float* cstar, hipStream_t stream) {
  TimingScope timing("bonus", stream);
  const dim3 grid(R, w.ns_b);
  if (bf16)
    hipLaunchKernelGGL(k_bonus<uint16_t>, grid, dim3(256), 0, stream, gamma, V, seed,
                       (const uint16_t*)T, w, cstar);
  else
    hipLaunchKernelGGL(k_bonus<float>, grid, dim3(256), 0, stream, gamma, V, seed, (const float*)T, w,
                       cstar);
  return hipGetLastError();
}

}  // namespace dspark
