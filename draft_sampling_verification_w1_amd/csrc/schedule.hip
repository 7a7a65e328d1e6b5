// schedule.hip -- prefix-survival products and the hardware-aware prefix
// scheduler (summary page §3.2.2, Algorithm 1 as described there):
//   a_{r,j} = prod_{i<=j} c_{r,i}
//   candidates (r, j) sorted by survival probability (key (-a, r, j), which
//   keeps each request's positions in order), B = sum(1 + l_r),
//   tau = sum(1 + sum a), Theta = tau * SPS(B); extend while Theta strictly
//   improves and stop at the first non-improvement (causal stop).
// One workgroup of 1024 threads: binary32 products per request, a stable
// radix sort of the candidates by survival (ties keep the (r, j) order), an
// exact integer scan of tau (units of 2^-38) and a parallel search for the
// first non-improving step.  Above 1024 candidates the stop is first sought
// in the head of the survival order alone (k_schedule).
//
// The same kernel serves the production variant (summary page §5.2): the
// capacity K of a later round is the candidate count with the largest Theta
// along the whole survival-ordered path (no early-stopping break, so a cliff
// in an irregular SPS curve does not end the search; the smallest count wins
// ties), and a round with a capacity handed to it verifies its first K
// candidates in current survival order (top-K).
#include "device_common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kMaxCand = 16384;
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kAlg1 = 0, kCapacity = 1, kTopK = 2;

__device__ __forceinline__ uint32_t survival_key_hi(float a) {
  const uint32_t b = __float_as_uint(a);
  if (b & 0x80000000u) return 0x3F800000u;      // -0 (and negative values) order as 0
  if (b > 0x3F800000u) return 0u;               // > 1 or NaN order as 1 (precondition broken)
  return 0x3F800000u - b;                       // ascending key = descending a
}

__device__ __forceinline__ float key_survival(uint64_t key) {
  return __uint_as_float(0x3F800000u - (uint32_t)(key >> 32));
}

// tau increment of a candidate: a rounded to the nearest multiple of 2^-38
__device__ __forceinline__ int64_t tau_unit(uint64_t key) {
  return (int64_t)__builtin_rint((double)key_survival(key) * 0x1p38);
}

// Exclusive prefix sum over the workgroup (every thread gets its offset and
// the total).
__device__ int64_t block_exclusive_scan(int64_t v, int64_t* wsum, int64_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int64_t before = 0;
  total = 0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) before += wsum[w];
    total += wsum[w];
  }
  return before + x - v;
}

// Largest value over the wave (every lane gets it), so that a workgroup
// maximum takes one LDS atomic per wave instead of one per thread on a single
// address.
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned long long y = __shfl_xor(x, off, 64);
    x = y > x ? y : x;
  }
  return x;
}

// Stable LSD radix sort of ks[0 .. EE * 1024) on the 30 bits of
// survival_key_hi (bits 32..61 of the key), 6 bits (64 digits) per pass.
// Wave w holds positions w*64EE + q*64 + lane (q < EE), so the order
// (wave, q, lane) is the position order.  A key's new place = the offset of
// (its digit, its wave) + the keys of that digit before it in the wave.
// Ballots of the digit bits give each lane the lanes of its q with the same
// digit; the lowest of them adds the group to the wave's counter of that
// digit (cnt[digit][wave], touched by this wave alone, in program order) and
// hands the previous count to the group.
template <int EE>
__device__ __forceinline__ void radix_sort(uint64_t* ks, int* cnt, int64_t* wsum) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int shift = 32; shift < 62; shift += 6) {
    uint64_t e[EE];
    int dig[EE], rank[EE];
    cnt[lane * kWaves + wave] = 0;  // digit = lane
#pragma unroll
    for (int q = 0; q < EE; ++q) {
      e[q] = ks[wave * 64 * EE + q * 64 + lane];
      const int d = (int)(e[q] >> shift) & 63;
      dig[q] = d;
      uint64_t same = ~0ull;
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        const uint64_t b = __ballot((d >> i) & 1);
        same &= ((d >> i) & 1) ? b : ~b;
      }
      const int before = __popcll(same & below);
      const int leader = __ffsll((unsigned long long)same) - 1;
      int prior = 0;
      if (before == 0) prior = atomicAdd(&cnt[d * kWaves + wave], __popcll(same));
      rank[q] = __shfl(prior, leader, 64) + before;
    }
    __syncthreads();
    int64_t total;
    // each thread scans and then overwrites its own entry: (digit, wave) order
    const int64_t off = block_exclusive_scan(cnt[tid], wsum, total);
    cnt[tid] = (int)off;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < EE; ++q) ks[cnt[dig[q] * kWaves + wave] + rank[q]] = e[q];
    __syncthreads();
  }
}

struct SchedShared {
  int64_t wsum[kWaves];
  int first_stop;
  int head_n;
  unsigned long long best_bits;
  unsigned long long umax, rest_bits;  // capacity head: largest tau unit outside, Theta bound
};

// The rest of a schedule once ks[0 .. m) holds the first m candidates of the
// survival order (thread t owns places EE t .. EE t + EE - 1; sp[q] is
// SPS(R + EE t + q), B = R + i candidates before place i): the exact tau scan,
// the stop (MODE), lengths, statistics and the Theta path.  With `head` set,
// ks holds only the first m of n candidates; if the stop is not decided
// within them the call writes nothing and returns false (for the capacity,
// `rest_bound` bounds Theta at every count past the head).  The per-request
// lengths are gathered in `len_area` (free once the keys are in registers).
template <int EE, int MODE>
__device__ __forceinline__ bool finish_schedule(const uint64_t* ks, int m, bool head, int R,
                                                int gamma, int n, const float* sps,
                                                const float (&sp)[EE + 1], float sps_r,
                                                void* len_area, SchedShared& sh, int32_t* lengths,
                                                double* stats, double* theta_path, int32_t* k_io,
                                                double rest_bound = 0.0) {
  constexpr bool kEarly = EE <= 8;
  const int tid = threadIdx.x;
  const int base = EE * tid;
  auto sps_at = [&](int q) -> float {
    if constexpr (kEarly) return sp[q];
    else return sps[R + base + q - 1];
  };
  if (tid == 0) {
    // kTopK: the count handed over (clamped to [0, n]); otherwise "no stop yet"
    int k0 = m;
    if constexpr (MODE == kTopK) k0 = min(max(k_io[0], 0), n);
    sh.first_stop = k0;
    // Theta >= 0 (a, SPS >= 0), so the bit patterns of the doubles order as the values
    sh.best_bits = (unsigned long long)__double_as_longlong((double)R * (double)sps_r);
  }
  uint64_t e[EE];
#pragma unroll
  for (int q = 0; q < EE; ++q) e[q] = base + q < m ? ks[base + q] : ~(uint64_t)0;

  // exact tau increments and their workgroup scan
  int64_t local = 0;
#pragma unroll
  for (int q = 0; q < EE; ++q) local += base + q < m ? tau_unit(e[q]) : 0;
  int64_t total;
  const int64_t offset = block_exclusive_scan(local, sh.wsum, total);
  const int64_t tau0 = (int64_t)R << 38;
  const double theta0 = (double)R * (double)sps_r;
  int64_t tau = tau0 + offset;  // before place base
  double best = 0.0;
  if constexpr (MODE == kAlg1) {
    int my_stop = m;
#pragma unroll
    for (int q = 0; q < EE; ++q) {
      const int i = base + q;
      if (i < m) {
        const double before = ldexp((double)tau, -38) * (double)sps_at(q);
        tau += tau_unit(e[q]);
        const double after = ldexp((double)tau, -38) * (double)sps_at(q + 1);
        if (!(after > before) && my_stop == m) my_stop = i;
      }
    }
    if (my_stop < m) atomicMin(&sh.first_stop, my_stop);
  } else if constexpr (MODE == kCapacity) {
    // the largest Theta after any count i + 1 = 1..n (count 0 seeded above),
    // then the smallest count that reaches it
    double th[EE];
    double mx = 0.0;
#pragma unroll
    for (int q = 0; q < EE; ++q) {
      const int i = base + q;
      th[q] = -1.0;
      if (i < m) {
        tau += tau_unit(e[q]);
        th[q] = ldexp((double)tau, -38) * (double)sps_at(q + 1);
        mx = fmax(mx, th[q]);
      }
    }
    const unsigned long long mb = wave_max_u64((unsigned long long)__double_as_longlong(mx));
    if ((tid & 63) == 0) atomicMax(&sh.best_bits, mb);
    __syncthreads();
    best = __longlong_as_double((long long)sh.best_bits);
    if (tid == 0 && (double)R * (double)sps_r == best) atomicMin(&sh.first_stop, 0);
#pragma unroll
    for (int q = 0; q < EE; ++q)
      if (th[q] == best) {
        atomicMin(&sh.first_stop, base + q + 1);
        break;
      }
  }
  __syncthreads();
  const int sel = sh.first_stop;
  // Algorithm 1 decides its stop at place sel from places 0..sel, so the head
  // must hold place sel; a top-K count needs places 0..K-1 only; the capacity
  // holds when no count past the head can exceed the head's best Theta (one
  // that only reaches it is not the smallest such count)
  bool outside = false;
  if constexpr (MODE == kAlg1) outside = sel >= m;
  else if constexpr (MODE == kTopK) outside = sel > m;
  else outside = rest_bound > best;
  if (head && outside) {
    __syncthreads();  // every thread has read first_stop and best_bits
    return false;
  }
  if constexpr (MODE == kCapacity) {
    if (tid == 0) k_io[0] = sel;
  }
  int* len = reinterpret_cast<int*>(len_area);
  for (int r = tid; r < R; r += kThreads) len[r] = 0;
  __syncthreads();

  // lengths: every selected candidate raises its request's length
  tau = tau0 + offset;
#pragma unroll
  for (int q = 0; q < EE; ++q) {
    const int i = base + q;
    if (i < m) {
      const uint32_t o = (uint32_t)e[q];
      tau += tau_unit(e[q]);
      const double th = ldexp((double)tau, -38) * (double)sps_at(q + 1);
      if (i < sel) atomicMax(&len[o / gamma], (int)(o % gamma) + 1);
      // Algorithm 1 records the path up to and including the stopping step;
      // the capacity search records all of it
      if (theta_path) theta_path[i + 1] = (MODE == kCapacity || i <= sel) ? th : NAN;
      if (i == sel - 1) {
        stats[0] = (double)(R + sel);
        stats[1] = ldexp((double)tau, -38);
        stats[2] = th;
        stats[3] = (double)sel;
      }
    }
  }
  if (theta_path)
    for (int i = m + tid; i < n; i += kThreads) theta_path[i + 1] = NAN;  // past the head
  __syncthreads();
  for (int r = tid; r < R; r += kThreads) lengths[r] = len[r];
  if (tid == 0) {
    if (theta_path) theta_path[0] = theta0;
    if (sel == 0) {
      stats[0] = (double)R;
      stats[1] = (double)R;
      stats[2] = theta0;
      stats[3] = 0.0;
    }
  }
  return true;
}

// E candidates per thread (E * 1024 >= R * gamma).  MODE: kAlg1 (causal
// stop), kCapacity (argmax of Theta over the whole path; K written to
// k_io[0]), kTopK (the first min(k_io[0], R*gamma) candidates).
//
// Head of the order (more than 1024 candidates): Algorithm 1 usually stops
// after a small part of the candidates (about one position per request where
// SPS bends at twice the batch), and a top-K count is usually small too.  A
// histogram of the top 10 key bits finds the longest run of leading buckets
// holding at most 1024 candidates; every other candidate has a larger key, so
// those candidates sorted are exactly the first places of the full order.
// They are sorted alone (one per thread), and the full sort runs only when the
// stop or the count lies beyond them.  The capacity (when no Theta path is
// asked for) takes the head's best Theta when no later count can exceed it:
// past the head, tau after c candidates is at most
// min(tau(m) + (c - m) u_max, tau(n)) with u_max the largest tau unit outside
// the head, and Theta(c) at most that bound times SPS(R + c), in the same
// monotone binary64 arithmetic as Theta itself.
template <int E, int MODE>
__global__ __launch_bounds__(kThreads) void k_schedule(int R, int gamma, const float* c,
                                                       const float* sps, float* a_out,
                                                       int32_t* lengths, double* stats,
                                                       double* theta_path, int32_t* k_io) {
  constexpr bool kHead = E >= 2;
  __shared__ uint64_t keys[kMaxCand];
  __shared__ int cnt[64 * kWaves];
  __shared__ uint64_t head_keys[kHead ? kThreads : 1];
  __shared__ int hist[kHead ? kThreads : 1];
  __shared__ SchedShared sh;
  const int tid = threadIdx.x;
  const int n = R * gamma;
  constexpr int npad = E * kThreads;
  const int base = E * tid;  // the thread's sorted places base .. base + E - 1

  // the stop test's table entries SPS(R + i) for i = base - 1 .. base + E - 1:
  // their places are known now, so the loads overlap the sort (at E = 16
  // the registers are short, and they are loaded where they are used)
  constexpr bool kEarly = E <= 8;
  float sp[E + 1];
  if constexpr (kEarly) {
#pragma unroll
    for (int q = 0; q <= E; ++q) sp[q] = (base + q <= n) ? sps[R + base + q - 1] : 0.0f;
  }
  // the head's places are tid (n > 1024 here, so both entries exist)
  float sp1[2] = {0.0f, 0.0f};
  if constexpr (kHead && kEarly) {
    sp1[0] = sps[R + tid - 1];
    sp1[1] = sps[R + tid];
  }
  const float sps_r = sps[R - 1];

  // prefix products, one request per thread (sequential binary32 multiplies;
  // a request's factors are fetched together, 16 at a time); the key of
  // candidate o = r * gamma + j sits at place o
  for (int r = tid; r < R; r += kThreads) {
    const int o0 = r * gamma;
    float acc = 1.0f;
    for (int j0 = 0; j0 < gamma; j0 += 16) {
      float cc[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) cc[u] = (j0 + u < gamma) ? c[o0 + j0 + u] : 1.0f;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (j0 + u < gamma) {
          const int o = o0 + j0 + u;
          acc = __fmul_rn(acc, cc[u]);
          a_out[o] = acc;
          keys[o] = ((uint64_t)survival_key_hi(acc) << 32) | (uint32_t)o;
        }
      }
    }
  }
  for (int p = n + tid; p < npad; p += kThreads) keys[p] = ~(uint64_t)0;  // after every real key
  if constexpr (kHead) hist[tid] = 0;
  __syncthreads();

  if constexpr (kHead) {
    if (MODE != kCapacity || theta_path == nullptr) {
      // bucket = key >> 52: the top 10 of the 30 survival-key bits
#pragma unroll
      for (int q = 0; q < E; ++q)
        if (base + q < n) atomicAdd(&hist[(int)(keys[base + q] >> 52)], 1);
      __syncthreads();
      int64_t tot;
      const int h = hist[tid];
      const int64_t incl = block_exclusive_scan(h, sh.wsum, tot) + h;  // candidates in buckets <= tid
      hist[tid] = incl <= kThreads ? 1 : 0;  // bucket in the head
      if (tid == 0) sh.head_n = 0;
      __syncthreads();
      const unsigned long long hn = wave_max_u64(incl <= kThreads ? (unsigned long long)incl : 0ull);
      if ((tid & 63) == 0 && hn > 0) atomicMax(&sh.head_n, (int)hn);
      __syncthreads();
      const int m = sh.head_n;
      if (m > 0) {
        // the head's keys in place order (equal keys keep their (r, j) order)
        bool in[E];
        int mine = 0;
        int64_t u_in = 0, u_all = 0;  // capacity: tau units of the head, of every candidate
        unsigned long long u_out = 0;  // and the largest outside the head
#pragma unroll
        for (int q = 0; q < E; ++q) {
          in[q] = base + q < n && hist[(int)(keys[base + q] >> 52)] != 0;
          mine += in[q] ? 1 : 0;
          if constexpr (MODE == kCapacity) {
            if (base + q < n) {
              const int64_t u = tau_unit(keys[base + q]);
              u_all += u;
              if (in[q]) u_in += u;
              else u_out = max(u_out, (unsigned long long)u);
            }
          }
        }
        int w = (int)block_exclusive_scan(mine, sh.wsum, tot);
#pragma unroll
        for (int q = 0; q < E; ++q)
          if (in[q]) head_keys[w++] = keys[base + q];
        if (tid >= m) head_keys[tid] = ~(uint64_t)0;
        __syncthreads();
        radix_sort<1>(head_keys, cnt, sh.wsum);
        if constexpr (!kEarly) {
          sp1[0] = sps[R + tid - 1];
          sp1[1] = sps[R + tid];
        }
        double rest_bound = 0.0;
        if constexpr (MODE == kCapacity) {
          if (tid == 0) {
            sh.umax = 0ull;
            sh.rest_bits = 0ull;
          }
          __syncthreads();
          u_out = wave_max_u64(u_out);
        if ((tid & 63) == 0) atomicMax(&sh.umax, u_out);
          int64_t t_in, t_all;
          block_exclusive_scan(u_in, sh.wsum, t_in);
          __syncthreads();  // the first scan's partial sums are read
          block_exclusive_scan(u_all, sh.wsum, t_all);
          const int64_t tau_head = ((int64_t)R << 38) + t_in, tau_all = ((int64_t)R << 38) + t_all;
          const int64_t um = (int64_t)sh.umax;
          double mx = 0.0;
          for (int cnt_c = m + 1 + tid; cnt_c <= n; cnt_c += kThreads) {
            const int64_t tb = min(tau_head + (int64_t)(cnt_c - m) * um, tau_all);
            mx = fmax(mx, ldexp((double)tb, -38) * (double)sps[R + cnt_c - 1]);
          }
          const unsigned long long mb = wave_max_u64((unsigned long long)__double_as_longlong(mx));
        if ((tid & 63) == 0) atomicMax(&sh.rest_bits, mb);
          __syncthreads();
          rest_bound = __longlong_as_double((long long)sh.rest_bits);
        }
        if (finish_schedule<1, MODE>(head_keys, m, true, R, gamma, n, sps, sp1, sps_r, keys, sh,
                                     lengths, stats, theta_path, k_io, rest_bound))
          return;
      }
    }
  }
  radix_sort<E>(keys, cnt, sh.wsum);
  finish_schedule<E, MODE>(keys, n, false, R, gamma, n, sps, sp, sps_r, keys, sh, lengths, stats,
                           theta_path, k_io);
}

}  // namespace

template <int MODE>
static void launch_mode(int R, int gamma, const float* c, const float* sps, float* a,
                        int32_t* lengths, double* stats, double* theta_path, int32_t* k_io,
                        hipStream_t stream) {
  const int64_t n = (int64_t)R * gamma;
  if (n <= kThreads)
    hipLaunchKernelGGL((k_schedule<1, MODE>), dim3(1), dim3(kThreads), 0, stream, R, gamma, c,
                       sps, a, lengths, stats, theta_path, k_io);
  else if (n <= 2 * kThreads)
    hipLaunchKernelGGL((k_schedule<2, MODE>), dim3(1), dim3(kThreads), 0, stream, R, gamma, c,
                       sps, a, lengths, stats, theta_path, k_io);
  else if (n <= 4 * kThreads)
    hipLaunchKernelGGL((k_schedule<4, MODE>), dim3(1), dim3(kThreads), 0, stream, R, gamma, c,
                       sps, a, lengths, stats, theta_path, k_io);
  else if (n <= 8 * kThreads)
    hipLaunchKernelGGL((k_schedule<8, MODE>), dim3(1), dim3(kThreads), 0, stream, R, gamma, c,
                       sps, a, lengths, stats, theta_path, k_io);
  else
    hipLaunchKernelGGL((k_schedule<16, MODE>), dim3(1), dim3(kThreads), 0, stream, R, gamma, c,
                       sps, a, lengths, stats, theta_path, k_io);
}

hipError_t launch_schedule(int R, int gamma, const float* c, const float* sps, float* a,
                           int32_t* lengths, double* stats, double* theta_path,
                           hipStream_t stream) {
  const int64_t n = (int64_t)R * gamma;
  if (n < 1 || n > kMaxCand) return hipErrorInvalidValue;
  TimingScope timing("schedule", stream);
  launch_mode<kAlg1>(R, gamma, c, sps, a, lengths, stats, theta_path, nullptr, stream);
  return hipGetLastError();
}

hipError_t launch_schedule_capacity(int R, int gamma, const float* c, const float* sps,
                                    float* a, int32_t* K, int32_t* lengths, double* stats,
                                    double* theta_path, hipStream_t stream) {
  const int64_t n = (int64_t)R * gamma;
  if (n < 1 || n > kMaxCand) return hipErrorInvalidValue;
  TimingScope timing("schedule_capacity", stream);
  launch_mode<kCapacity>(R, gamma, c, sps, a, lengths, stats, theta_path, K, stream);
  return hipGetLastError();
}

hipError_t launch_schedule_topk(int R, int gamma, const float* c, const int32_t* K,
                                const float* sps, float* a, int32_t* lengths, double* stats,
                                hipStream_t stream) {
  const int64_t n = (int64_t)R * gamma;
  if (n < 1 || n > kMaxCand) return hipErrorInvalidValue;
  TimingScope timing("schedule_topk", stream);
  launch_mode<kTopK>(R, gamma, c, sps, a, lengths, stats, nullptr, const_cast<int32_t*>(K),
                     stream);
  return hipGetLastError();
}

}  // namespace dspark
