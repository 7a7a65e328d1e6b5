// schedule.hip -- prefix-survival products and the hardware-aware prefix
// scheduler (summary page §3.2.2, Algorithm 1 as described there):
//   a_{r,j} = prod_{i<=j} c_{r,i}
//   candidates (r, j) sorted by survival probability (key (-a, r, j), which
//   keeps each request's positions in order), B = sum(1 + l_r),
//   tau = sum(1 + sum a), Theta = tau * SPS(B); extend while Theta strictly
//   improves and stop at the first non-improvement (causal stop).
// One workgroup of 1024 threads: binary32 products per request, a merge sort
// of the 64-bit keys, an exact integer scan of tau (units of 2^-38) and a
// parallel search for the first non-improving step.  Because every factor c
// lies in [0, 1], a request's products never increase with j, so its keys are
// already an ascending run; the sort only merges runs pairwise (each key finds
// its place by a binary search in the partner run).
#include "device_common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kMaxCand = 16384;
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

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

template <int E>
__global__ __launch_bounds__(kThreads) void k_schedule(int R, int gamma, const float* c,
                                                       const float* sps, float* a_out,
                                                       int32_t* lengths, double* stats,
                                                       double* theta_path) {
  __shared__ uint64_t keys[kMaxCand];
  __shared__ int64_t wsum[kWaves];
  __shared__ int first_stop;
  const int tid = threadIdx.x;
  const int n = R * gamma;

  // prefix products, one request per thread (sequential binary32 multiplies;
  // a request's factors are fetched together, 16 at a time)
  for (int r = tid; r < R; r += kThreads) {
    const int o0 = r * gamma;
    float acc = 1.0f;
    uint64_t prev = 0;
    bool ascending = true;
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
          const uint64_t key = ((uint64_t)survival_key_hi(acc) << 32) | (uint32_t)o;
          ascending = ascending && (o == o0 || key > prev);
          prev = key;
          keys[o] = key;
        }
      }
    }
    // a factor above 1 (a c* rounded up past 1, say) can break the run: sort
    // the request's own keys (insertion sort, the run is nearly in order)
    if (!ascending) {
      for (int i = o0 + 1; i < o0 + gamma; ++i) {
        const uint64_t x = keys[i];
        int j = i - 1;
        while (j >= o0 && keys[j] > x) {
          keys[j + 1] = keys[j];
          --j;
        }
        keys[j + 1] = x;
      }
    }
    lengths[r] = 0;
  }
  if (tid == 0) first_stop = n;
  __syncthreads();

  // merge runs pairwise: run m covers [m*L, min((m+1)*L, n)); an element of
  // run m moves to (start of the pair) + (its place in run m) + (keys of the
  // partner run below it).  Keys are distinct, so the order is total.
  const int base = E * tid;
  uint64_t e[E];
  int run0[E];  // run of each of the thread's positions at the first level
#pragma unroll
  for (int q = 0; q < E; ++q) run0[q] = (base + q) / gamma;
  int level = 0;
  for (int L = gamma; L < n; L <<= 1, ++level) {
    // binary search of each key in the partner run (fixed number of steps)
    int dest[E], lo[E], len[E];
#pragma unroll
    for (int q = 0; q < E; ++q) {
      const int p = base + q;
      dest[q] = 0;
      lo[q] = 0;
      len[q] = 0;
      if (p < n) {
        e[q] = keys[p];
        const int m = run0[q] >> level;
        const int pair = (m >> 1) * 2 * L;
        const int plo = (m & 1) ? pair : min(pair + L, n);
        const int phi = (m & 1) ? pair + L : min(pair + 2 * L, n);
        dest[q] = pair + (p - m * L) - plo;  // + index of the first partner key >= e[q]
        lo[q] = plo;
        len[q] = phi - plo;
      }
    }
    for (int steps = 32 - __builtin_clz(L); steps > 0; --steps) {
#pragma unroll
      for (int q = 0; q < E; ++q) {
        if (len[q] > 0) {
          const int half = len[q] >> 1;
          if (keys[lo[q] + half] < e[q]) {
            lo[q] += half + 1;
            len[q] -= half + 1;
          } else {
            len[q] = half;
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < E; ++q)
      if (base + q < n) keys[dest[q] + lo[q]] = e[q];
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < E; ++q) e[q] = base + q < n ? keys[base + q] : ~(uint64_t)0;

  // exact tau increments and their workgroup scan
  int64_t local = 0;
#pragma unroll
  for (int q = 0; q < E; ++q) local += base + q < n ? tau_unit(e[q]) : 0;
  int64_t total;
  const int64_t offset = block_exclusive_scan(local, wsum, total);
  const int64_t tau0 = (int64_t)R << 38;
  const double theta0 = (double)R * (double)sps[R - 1];
  int64_t tau = tau0 + offset;  // before element base
  int my_stop = n;
#pragma unroll
  for (int q = 0; q < E; ++q) {
    const int i = base + q;
    if (i < n) {
      const double before = ldexp((double)tau, -38) * (double)sps[R + i - 1];
      tau += tau_unit(e[q]);
      const double after = ldexp((double)tau, -38) * (double)sps[R + i];
      if (!(after > before) && my_stop == n) my_stop = i;
    }
  }
  if (my_stop < n) atomicMin(&first_stop, my_stop);
  __syncthreads();
  const int sel = first_stop;

  // lengths: every selected candidate raises its request's length
  tau = tau0 + offset;
#pragma unroll
  for (int q = 0; q < E; ++q) {
    const int i = base + q;
    if (i < n) {
      const uint32_t o = (uint32_t)e[q];
      tau += tau_unit(e[q]);
      const double th = ldexp((double)tau, -38) * (double)sps[R + i];
      if (i < sel) atomicMax(&lengths[o / gamma], (int)(o % gamma) + 1);
      if (theta_path) theta_path[i + 1] = (i <= sel) ? th : NAN;
      if (i == sel - 1) {
        stats[0] = (double)(R + sel);
        stats[1] = ldexp((double)tau, -38);
        stats[2] = th;
        stats[3] = (double)sel;
      }
    }
  }
  if (tid == 0) {
    if (theta_path) theta_path[0] = theta0;
    if (sel == 0) {
      stats[0] = (double)R;
      stats[1] = (double)R;
      stats[2] = theta0;
      stats[3] = 0.0;
    }
  }
}

}  // namespace

hipError_t launch_schedule(int R, int gamma, const float* c, const float* sps, float* a,
                           int32_t* lengths, double* stats, double* theta_path,
                           hipStream_t stream) {
  const int64_t n = (int64_t)R * gamma;
  if (n < 1 || n > kMaxCand) return hipErrorInvalidValue;
  TimingScope timing("schedule", stream);
  if (n <= 4 * kThreads)
    hipLaunchKernelGGL(k_schedule<4>, dim3(1), dim3(kThreads), 0, stream, R, gamma, c, sps, a,
                       lengths, stats, theta_path);
  else if (n <= 8 * kThreads)
    hipLaunchKernelGGL(k_schedule<8>, dim3(1), dim3(kThreads), 0, stream, R, gamma, c, sps, a,
                       lengths, stats, theta_path);
  else
    hipLaunchKernelGGL(k_schedule<16>, dim3(1), dim3(kThreads), 0, stream, R, gamma, c, sps, a,
                       lengths, stats, theta_path);
  return hipGetLastError();
}

}  // namespace dspark
