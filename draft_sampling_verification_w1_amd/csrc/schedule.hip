// schedule.hip -- prefix-survival products and the hardware-aware prefix
// scheduler (summary page §3.2.2, Algorithm 1 as described there):
//   a_{r,j} = prod_{i<=j} c_{r,i}
//   candidates (r, j) sorted by survival probability (key (-a, r, j), which
//   keeps each request's positions in order), B = sum(1 + l_r),
//   tau = sum(1 + sum a), Theta = tau * SPS(B); extend while Theta strictly
//   improves and stop at the first non-improvement (causal stop).
// One workgroup: binary32 products per request, a bitonic sort of the 64-bit
// keys in LDS, an exact integer scan of tau (units of 2^-38) and a parallel
// search for the first non-improving step.
#include "device_common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kMaxCand = 16384;
constexpr int kThreads = 1024;

__device__ __forceinline__ uint32_t survival_key_hi(float a) {
  const uint32_t b = __float_as_uint(a);
  if (b & 0x80000000u) return 0x3F800000u;      // -0 (and negative values) order as 0
  if (b > 0x3F800000u) return 0u;               // > 1 or NaN order as 1 (precondition broken)
  return 0x3F800000u - b;                       // ascending key = descending a
}

__global__ __launch_bounds__(kThreads) void k_schedule(int R, int gamma, const float* c,
                                                       const float* sps, float* a_out,
                                                       int32_t* lengths, double* stats,
                                                       double* theta_path) {
  __shared__ uint64_t keys[kMaxCand];
  __shared__ int64_t scan[kThreads];
  __shared__ int first_stop;
  const int tid = threadIdx.x;
  const int n = R * gamma;
  int npad = 1;
  while (npad < n) npad <<= 1;

  // prefix products, one request per thread (sequential binary32 multiplies)
  for (int r = tid; r < R; r += kThreads) {
    float acc = 1.0f;
    for (int j = 0; j < gamma; ++j) {
      const int o = r * gamma + j;
      acc = __fmul_rn(acc, c[o]);
      a_out[o] = acc;
      keys[o] = ((uint64_t)survival_key_hi(acc) << 32) | (uint32_t)o;
    }
    lengths[r] = 0;
  }
  for (int i = n + tid; i < npad; i += kThreads) keys[i] = ~(uint64_t)0;
  if (tid == 0) first_stop = n;
  __syncthreads();

  // bitonic sort, ascending
  for (int k = 2; k <= npad; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < npad; i += kThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = keys[i], y = keys[ixj];
          const bool asc = (i & k) == 0;
          if ((x > y) == asc) {
            keys[i] = y;
            keys[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }

  // exact tau increments and their block scan (contiguous ranges per thread)
  const int per = (n + kThreads - 1) / kThreads;
  const int i0 = min(tid * per, n), i1 = min(i0 + per, n);
  int64_t local = 0;
  for (int i = i0; i < i1; ++i) {
    const float a = __uint_as_float(0x3F800000u - (uint32_t)(keys[i] >> 32));
    local += (int64_t)__builtin_rint((double)a * 0x1p38);
  }
  scan[tid] = local;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int64_t v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const int64_t tau0 = (int64_t)R << 38;
  const double theta0 = (double)R * (double)sps[R - 1];
  int64_t tau = tau0 + scan[tid] - local;  // before element i0
  int my_stop = n;
  for (int i = i0; i < i1; ++i) {
    const float a = __uint_as_float(0x3F800000u - (uint32_t)(keys[i] >> 32));
    const int64_t unit = (int64_t)__builtin_rint((double)a * 0x1p38);
    const double before = ldexp((double)tau, -38) * (double)sps[R + i - 1];
    tau += unit;
    const double after = ldexp((double)tau, -38) * (double)sps[R + i];
    if (!(after > before) && my_stop == n) my_stop = i;
  }
  if (my_stop < n) atomicMin(&first_stop, my_stop);
  __syncthreads();
  const int sel = first_stop;

  // lengths: every selected candidate raises its request's length
  tau = tau0 + scan[tid] - local;
  for (int i = i0; i < i1; ++i) {
    const uint32_t o = (uint32_t)keys[i];
    const float a = __uint_as_float(0x3F800000u - (uint32_t)(keys[i] >> 32));
    tau += (int64_t)__builtin_rint((double)a * 0x1p38);
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
  TimingScope timing("schedule", stream);
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(kThreads), 0, stream, R, gamma, c, sps, a, lengths,
                     stats, theta_path);
  return hipGetLastError();
}

}  // namespace dspark
