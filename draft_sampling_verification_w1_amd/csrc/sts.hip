// sts.hip -- Sequential Temperature Scaling fit (summary page §3.2.1): the
// cumulative prefix survival is calibrated on held-out rollouts by a
// left-to-right one-dimensional grid search, each position's temperature
// chosen to minimise that position's Expected Calibration Error with the
// earlier positions' temperatures fixed.
//
// Per position j (three launches, in order on the stream):
//   k_sts_hist   : one workgroup per (candidate temperature, chunk of
//                  rollouts); survival a = fl32(a_{j-1} * fl32(sigmoid(s / T)))
//                  binned into `bins` equal-width bins of [0, 1]; per bin the
//                  sum of (label - a) in units of 2^-40 (exact integers, so
//                  the result does not depend on the order of the sums);
//                  workgroup sums in LDS, then one global atomic per bin;
//   k_sts_choose : one workgroup; N * ECE of every candidate = sum of the
//                  bins' absolute values; the smallest wins (lowest grid
//                  index on ties); the ECE at T = 1 is kept beside it;
//   k_sts_apply  : the chosen temperature's survival for every rollout.
#include "device_common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kStsThreads = 256;

__device__ __forceinline__ float sts_survival(float prev, double s, double T) {
  const float c = (float)(1.0 / (1.0 + exp(-s / T)));
  return __fmul_rn(prev, c);
}

__device__ __forceinline__ int64_t sts_units(float a) {
  return (int64_t)rint(ldexp((double)a, 40));
}

// acc: [gamma][G + 1][bins] int64 (candidate G is T = 1)
__global__ __launch_bounds__(kStsThreads) void k_sts_hist(int N, int gamma, int j, const double* s,
                                                          const uint8_t* y, int G,
                                                          const double* grid, int bins,
                                                          const float* a, int64_t* acc) {
  __shared__ unsigned long long hist[kStsMaxBins];
  const int g = blockIdx.x;
  const double T = g < G ? grid[g] : 1.0;
  for (int b = threadIdx.x; b < bins; b += kStsThreads) hist[b] = 0ull;
  __syncthreads();
  const int chunk = (N + gridDim.y - 1) / gridDim.y;
  const int n0 = blockIdx.y * chunk;
  const int n1 = min(N, n0 + chunk);
  for (int n = n0 + threadIdx.x; n < n1; n += kStsThreads) {
    const int64_t o = (int64_t)n * gamma + j;
    const float prev = j > 0 ? a[o - 1] : 1.0f;
    const float an = sts_survival(prev, s[o], T);
    const int b = min((int)floor((double)an * (double)bins), bins - 1);
    const int64_t v = ((int64_t)(y[o] != 0) << 40) - sts_units(an);
    atomicAdd(&hist[max(b, 0)], (unsigned long long)v);
  }
  __syncthreads();
  int64_t* dst = acc + ((int64_t)j * (G + 1) + g) * bins;
  for (int b = threadIdx.x; b < bins; b += kStsThreads)
    if (hist[b] != 0ull) atomicAdd(reinterpret_cast<unsigned long long*>(dst + b), hist[b]);
}

__global__ __launch_bounds__(kStsThreads) void k_sts_choose(int gamma, int j, int G,
                                                            const double* grid, int bins,
                                                            const int64_t* acc, int32_t* chosen,
                                                            float* temps, int64_t* ece_units,
                                                            int64_t* ece1_units) {
  __shared__ unsigned long long best_e;
  __shared__ int best_g;
  if (threadIdx.x == 0) {
    best_e = ~0ull;
    best_g = G;
  }
  __syncthreads();
  const int64_t* base = acc + (int64_t)j * (G + 1) * bins;
  auto ece = [&](int g) {
    int64_t e = 0;
    for (int b = 0; b < bins; ++b) {
      const int64_t x = base[(int64_t)g * bins + b];
      e += x < 0 ? -x : x;
    }
    return e;
  };
  for (int g = threadIdx.x; g < G; g += kStsThreads) atomicMin(&best_e, (unsigned long long)ece(g));
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += kStsThreads)
    if ((unsigned long long)ece(g) == best_e) atomicMin(&best_g, g);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int gb = min(best_g, G - 1);  // always < G: some candidate attains the minimum
    chosen[j] = gb;
    temps[j] = (float)grid[gb];
    ece_units[j] = (int64_t)best_e;
    ece1_units[j] = ece(G);
  }
}

__global__ __launch_bounds__(kStsThreads) void k_sts_apply(int N, int gamma, int j, const double* s,
                                                           const double* grid,
                                                           const int32_t* chosen, float* a) {
  const int n = blockIdx.x * kStsThreads + threadIdx.x;
  if (n >= N) return;
  const int64_t o = (int64_t)n * gamma + j;
  const float prev = j > 0 ? a[o - 1] : 1.0f;
  a[o] = sts_survival(prev, s[o], grid[chosen[j]]);
}

__global__ void k_fill_i64(int64_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace

size_t sts_workspace_bytes(int gamma, int G, int bins) {
  return (size_t)gamma * (G + 1) * bins * sizeof(int64_t) + 256 + (size_t)gamma * sizeof(int32_t);
}

hipError_t launch_sts_fit(int N, int gamma, const double* s, const uint8_t* y, int G,
                          const double* grid, int bins, float* temps, int64_t* ece_units,
                          int64_t* ece1_units, float* a, void* ws, hipStream_t stream) {
  TimingScope timing("sts_fit", stream);
  int64_t* acc = static_cast<int64_t*>(ws);
  const size_t acc_bytes = (size_t)gamma * (G + 1) * bins * sizeof(int64_t);
  int32_t* chosen = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + ((acc_bytes + 255) & ~size_t(255)));
  const int64_t n_acc = (int64_t)gamma * (G + 1) * bins;
  const int64_t fill_blocks = (n_acc + 255) / 256 < 1024 ? (n_acc + 255) / 256 : 1024;
  hipLaunchKernelGGL(k_fill_i64, dim3((unsigned)fill_blocks), dim3(256), 0, stream, acc, n_acc);
  // about 2048 workgroups per histogram pass, at least 256 rollouts each
  const int chunks = max(1, min((N + kStsThreads - 1) / kStsThreads, 2048 / (G + 1)));
  for (int j = 0; j < gamma; ++j) {
    hipLaunchKernelGGL(k_sts_hist, dim3(G + 1, chunks), dim3(kStsThreads), 0, stream, N, gamma, j,
                       s, y, G, grid, bins, a, acc);
    hipLaunchKernelGGL(k_sts_choose, dim3(1), dim3(kStsThreads), 0, stream, gamma, j, G, grid, bins,
                       acc, chosen, temps, ece_units, ece1_units);
    hipLaunchKernelGGL(k_sts_apply, dim3((N + kStsThreads - 1) / kStsThreads), dim3(kStsThreads), 0,
                       stream, N, gamma, j, s, grid, chosen, a);
  }
  return hipGetLastError();
}

}  // namespace dspark
