// acceptance.hip -- static-threshold verify lengths and acceptance statistics.
//
// Summary page §4.3.3: the static-threshold experiment verifies, per request,
// the prefix whose estimated survival a_{r,j} = prod_{i<=j} c_{r,i} stays at
// or above a fixed threshold; l_r is the largest j with a_{r,i} >= theta for
// every i <= j.  Summary page §4.3.1: the acceptance at position k is counted
// only over rollouts whose earlier draft tokens were all accepted.
//
// Both are small: one request per thread for the lengths; for the statistics
// one workgroup for the mask and one per threshold of the sweep (no memset,
// so a captured graph can replay it).
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

// Workgroup 0: per request, p = its leading accepted positions (mask 1);
// positions 1..p count as reached and accepted, and position p + 1 as reached
// when it was verified and rejected (mask 0).  Workgroup 1 + g: threshold g of
// the sweep, sum_r l_r(theta) and sum_r min(n_r, l_r(theta)).
__global__ __launch_bounds__(kStatThreads) void k_acceptance_stats(
    int R, int gamma, const uint8_t* mask, const float* a, const int32_t* n_accept,
    const double* thresholds, int n_thr, int64_t* reached, int64_t* accepted,
    int64_t* sweep_verified, int64_t* sweep_accepted) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
    if (!mask) return;
    // s_acc[p]: requests whose accepted prefix is p (0..gamma); s_rej[p]: those
    // of them that were verified and rejected at position p + 1
    __shared__ unsigned long long s_acc[65], s_rej[65];
    if (tid < 65) s_acc[tid] = s_rej[tid] = 0;
    __syncthreads();
    for (int r = tid; r < R; r += kStatThreads) {
      const uint8_t* m = mask + (int64_t)r * gamma;
      int p = 0;
      while (p < gamma && m[p] == 1) ++p;
      atomicAdd(&s_acc[p], 1ull);  // p <= gamma <= 64
      if (p < gamma && m[p] == 0) atomicAdd(&s_rej[p], 1ull);
    }
    __syncthreads();
    if (tid < gamma) {
      // reached[k] = #(p > k) + #(p = k rejected); accepted[k] = #(p > k)
      unsigned long long above = 0;
      for (int q = tid + 1; q <= gamma; ++q) above += s_acc[q];
      reached[tid] = (int64_t)(above + s_rej[tid]);
      accepted[tid] = (int64_t)above;
    }
    return;
  }
  const int g = blockIdx.x - 1;
  if (g >= n_thr) return;
  const double th = thresholds[g];
  unsigned long long ver = 0, acc = 0;
  for (int r = tid; r < R; r += kStatThreads) {
    const float* ar = a + (int64_t)r * gamma;
    int l = 0;
    while (l < gamma && (double)ar[l] >= th) ++l;
    const int n = n_accept[r];
    ver += (unsigned long long)l;
    acc += (unsigned long long)(n < l ? n : l);
  }
  __shared__ unsigned long long s_ver[kStatThreads / 64], s_sac[kStatThreads / 64];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    ver += __shfl_xor(ver, off, 64);
    acc += __shfl_xor(acc, off, 64);
  }
  if ((tid & 63) == 0) {
    s_ver[tid >> 6] = ver;
    s_sac[tid >> 6] = acc;
  }
  __syncthreads();
  if (tid == 0) {
    unsigned long long v = 0, c = 0;
    for (int w = 0; w < kStatThreads / 64; ++w) {
      v += s_ver[w];
      c += s_sac[w];
    }
    sweep_verified[g] = (int64_t)v;
    sweep_accepted[g] = (int64_t)c;
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
  hipLaunchKernelGGL(k_acceptance_stats, dim3(1 + n_thr), dim3(kStatThreads), 0, stream, R, gamma, mask,
                     a, n_accept, thresholds, n_thr, reached, accepted, sweep_verified,
                     sweep_accepted);
  return hipGetLastError();
}

}  // namespace dspark
