// acceptance.hip -- static-threshold verify lengths and acceptance statistics.
//
// Summary page §4.3.3: the static-threshold experiment verifies, per request,
// the prefix whose estimated survival a_{r,j} = prod_{i<=j} c_{r,i} stays at
// or above a fixed threshold; l_r is the largest j with a_{r,i} >= theta for
// every i <= j.  Summary page §4.3.1: the acceptance at position k is counted
// only over rollouts whose earlier draft tokens were all accepted.
//
// Both are small: one request per thread for the lengths, and one workgroup
// for the statistics (no memset, so a captured graph can replay it).
#include "device_common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kStatThreads = 1024;

// a = binary32 prefix products of c; l_r = leading positions with a >= theta
// (compared in binary64).
__global__ __launch_bounds__(256) void k_threshold(int R, int gamma, const float* c,
                                                   double theta, float* a, int32_t* lengths) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int64_t o0 = (int64_t)r * gamma;
  float acc = 1.0f;
  int l = 0;
  bool run = true;
  for (int j = 0; j < gamma; ++j) {
    acc = __fmul_rn(acc, c[o0 + j]);
    a[o0 + j] = acc;
    run = run && ((double)acc >= theta);
    l += run ? 1 : 0;
  }
  lengths[r] = l;
}

// One workgroup.  Per request: p = its leading accepted positions (mask 1);
// positions 1..p count as reached and accepted, and position p + 1 as reached
// when it was verified and rejected (mask 0).  The threshold sweep counts, per
// threshold, sum_r l_r(theta) and sum_r min(n_r, l_r(theta)).
__global__ __launch_bounds__(kStatThreads) void k_acceptance_stats(
    int R, int gamma, const uint8_t* mask, const float* a, const int32_t* n_accept,
    const double* thresholds, int n_thr, int64_t* reached, int64_t* accepted,
    int64_t* sweep_verified, int64_t* sweep_accepted) {
  // s_acc[p]: requests whose accepted prefix is p (0..gamma); s_rej[p]: those
  // of them that were verified and rejected at position p + 1
  __shared__ unsigned long long s_acc[65], s_rej[65];
  __shared__ unsigned long long s_ver[kMaxThresholds], s_sac[kMaxThresholds];
  const int tid = threadIdx.x;
  if (tid < 65) s_acc[tid] = s_rej[tid] = 0;
  for (int g = tid; g < n_thr; g += kStatThreads) s_ver[g] = s_sac[g] = 0;
  __syncthreads();
  if (mask) {
    for (int r = tid; r < R; r += kStatThreads) {
      const uint8_t* m = mask + (int64_t)r * gamma;
      int p = 0;
      while (p < gamma && m[p] == 1) ++p;
      atomicAdd(&s_acc[p], 1ull);  // p <= gamma <= 64
      if (p < gamma && m[p] == 0) atomicAdd(&s_rej[p], 1ull);
    }
  }
  // sweep: one (request, threshold) pair per step of the loop
  if (n_thr > 0) {
    const int64_t total = (int64_t)R * n_thr;
    for (int64_t idx = tid; idx < total; idx += kStatThreads) {
      const int r = (int)(idx / n_thr), g = (int)(idx - (int64_t)r * n_thr);
      const double th = thresholds[g];
      const float* ar = a + (int64_t)r * gamma;
      int l = 0;
      while (l < gamma && (double)ar[l] >= th) ++l;
      const int n = n_accept[r];
      atomicAdd(&s_ver[g], (unsigned long long)l);
      atomicAdd(&s_sac[g], (unsigned long long)(n < l ? n : l));
    }
  }
  __syncthreads();
  if (mask && tid < gamma) {
    // reached[k] = #(p > k) + #(p = k rejected); accepted[k] = #(p > k)
    unsigned long long above = 0;
    for (int q = tid + 1; q <= gamma; ++q) above += s_acc[q];
    reached[tid] = (int64_t)(above + s_rej[tid]);
    accepted[tid] = (int64_t)above;
  }
  for (int g = tid; g < n_thr; g += kStatThreads) {
    sweep_verified[g] = (int64_t)s_ver[g];
    sweep_accepted[g] = (int64_t)s_sac[g];
  }
}

}  // namespace

hipError_t launch_threshold(int R, int gamma, const float* c, double theta, float* a,
                            int32_t* lengths, hipStream_t stream) {
  TimingScope timing("threshold", stream);
  hipLaunchKernelGGL(k_threshold, dim3((R + 255) / 256), dim3(256), 0, stream, R, gamma, c, theta,
                     a, lengths);
  return hipGetLastError();
}

hipError_t launch_acceptance_stats(int R, int gamma, const uint8_t* mask, const float* a,
                                   const int32_t* n_accept, const double* thresholds, int n_thr,
                                   int64_t* reached, int64_t* accepted, int64_t* sweep_verified,
                                   int64_t* sweep_accepted, hipStream_t stream) {
  if (n_thr < 0 || n_thr > kMaxThresholds || gamma < 1 || gamma > 64) return hipErrorInvalidValue;
  TimingScope timing("acceptance_stats", stream);
  hipLaunchKernelGGL(k_acceptance_stats, dim3(1), dim3(kStatThreads), 0, stream, R, gamma, mask,
                     a, n_accept, thresholds, n_thr, reached, accepted, sweep_verified,
                     sweep_accepted);
  return hipGetLastError();
}

}  // namespace dspark
