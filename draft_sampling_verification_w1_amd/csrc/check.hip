// check.hip -- device-side check of the values the host cannot see (token ids,
// confidences, non-finite logits and weights): a debugging aid off the hot
// path.  Every test is on bit patterns, so that it holds whatever the
// compiler assumes about NaN.
#include "device_common.h"
#include "kernels.h"

namespace dspark {

namespace {

enum CheckKind {
  kIdRange = 0,    // int32 outside [0, V)
  kNanPosInf = 1,  // NaN or +inf (a logit of -inf masks an entry)
  kNonFinite = 2,  // NaN or +-inf
  kUnitRange = 3,  // binary32 outside [0, 1], or NaN
};

__device__ __forceinline__ bool bad_f32(uint32_t b, int kind) {
  const bool nan = (b & 0x7FFFFFFFu) > 0x7F800000u;
  if (kind == kNanPosInf) return nan || b == 0x7F800000u;
  if (kind == kNonFinite) return (b & 0x7F800000u) == 0x7F800000u;
  // [0, 1]: +0, -0 and the positive values up to 1.0f
  return nan || (b > 0x3F800000u && b != 0x80000000u);
}

__device__ __forceinline__ bool bad_bf16(uint32_t h, int kind) {
  return bad_f32(h << 16, kind);
}

template <int KIND, int ESIZE>
__device__ __forceinline__ int count_word(uint32_t w, int V) {
  if constexpr (KIND == kIdRange) {
    const int x = (int)w;
    return (x < 0 || x >= V) ? 1 : 0;
  } else if constexpr (ESIZE == 2) {
    return (bad_bf16(w & 0xFFFFu, KIND) ? 1 : 0) + (bad_bf16(w >> 16, KIND) ? 1 : 0);
  } else {
    return bad_f32(w, KIND) ? 1 : 0;
  }
}

// Counts the bad entries among n elements of ESIZE bytes; one atomic per
// workgroup.  16-byte loads over the aligned body, element loads at the ends.
template <int KIND, int ESIZE>
__global__ __launch_bounds__(256) void k_count(const void* p, int64_t n, int V,
                                               unsigned long long* count) {
  const uint8_t* base = static_cast<const uint8_t*>(p);
  const int64_t bytes = n * ESIZE;
  const uintptr_t a = reinterpret_cast<uintptr_t>(base);
  int64_t head = (int64_t)(((a + 15) & ~(uintptr_t)15) - a);  // bytes before the first 16-byte boundary
  if (head > bytes) head = bytes;
  const int64_t nvec = (bytes - head) / 16;
  const int64_t tail0 = head + nvec * 16;
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nthreads = (int64_t)gridDim.x * 256;
  unsigned long long c = 0;
  const u32x4* body = reinterpret_cast<const u32x4*>(base + head);
  for (int64_t i = tid; i < nvec; i += nthreads) {
    const u32x4 v = __builtin_nontemporal_load(body + i);
    c += count_word<KIND, ESIZE>(v.x, V) + count_word<KIND, ESIZE>(v.y, V) +
         count_word<KIND, ESIZE>(v.z, V) + count_word<KIND, ESIZE>(v.w, V);
  }
  // the unaligned head and tail, one element per thread (ESIZE divides the
  // offsets: element pointers are ESIZE-aligned)
  const int64_t nhead = head / ESIZE, ntail = (bytes - tail0) / ESIZE;
  for (int64_t i = tid; i < nhead + ntail; i += nthreads) {
    const int64_t off = i < nhead ? i * ESIZE : tail0 + (i - nhead) * ESIZE;
    const uint32_t w = ESIZE == 2 ? (uint32_t)*reinterpret_cast<const uint16_t*>(base + off)
                                  : *reinterpret_cast<const uint32_t*>(base + off);
    c += ESIZE == 2 ? (bad_bf16(w, KIND) ? 1 : 0) : count_word<KIND, ESIZE>(w, V);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
  __shared__ unsigned long long wsum[4];
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long s = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (s) atomicAdd(count, s);
  }
}

__global__ void k_zero_counts(unsigned long long* counts, int n) {
  if ((int)threadIdx.x < n) counts[threadIdx.x] = 0ull;
}

template <int KIND, int ESIZE>
hipError_t count(const void* p, int64_t n, int V, unsigned long long* out, hipStream_t s) {
  if (p == nullptr || n <= 0) return hipSuccess;
  const int64_t vec = (n * ESIZE) / 16 + 1;
  const int64_t want = (vec + 255) / 256;
  const int grid = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL((k_count<KIND, ESIZE>), dim3(grid), dim3(256), 0, s, p, n, V, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_check_inputs(bool bf16, int R, int gamma, int V, const void* U, const void* T,
                               const void* W1, const void* W2, const int32_t* anchors,
                               const int32_t* tokens, const float* c, int64_t* counts,
                               hipStream_t s) {
  unsigned long long* out = reinterpret_cast<unsigned long long*>(counts);
  hipLaunchKernelGGL(k_zero_counts, dim3(1), dim3(64), 0, s, out, kCheckCounts);
  hipError_t e = hipGetLastError();
  const int64_t rows = (int64_t)R * gamma;
  if (e == hipSuccess) e = count<kIdRange, 4>(anchors, R, V, out + 0, s);
  if (e == hipSuccess) e = count<kIdRange, 4>(tokens, rows, V, out + 1, s);
  if (bf16) {
    if (e == hipSuccess) e = count<kNanPosInf, 2>(U, rows * V, V, out + 2, s);
    if (e == hipSuccess) e = count<kNanPosInf, 2>(T, (int64_t)R * (gamma + 1) * V, V, out + 3, s);
    if (e == hipSuccess) e = count<kNonFinite, 2>(W1, (int64_t)V * kRank, V, out + 4, s);
    if (e == hipSuccess) e = count<kNonFinite, 2>(W2, (int64_t)kRank * V, V, out + 4, s);
  } else {
    if (e == hipSuccess) e = count<kNanPosInf, 4>(U, rows * V, V, out + 2, s);
    if (e == hipSuccess) e = count<kNanPosInf, 4>(T, (int64_t)R * (gamma + 1) * V, V, out + 3, s);
    if (e == hipSuccess) e = count<kNonFinite, 4>(W1, (int64_t)V * kRank, V, out + 4, s);
    if (e == hipSuccess) e = count<kNonFinite, 4>(W2, (int64_t)kRank * V, V, out + 4, s);
  }
  if (e == hipSuccess) e = count<kUnitRange, 4>(c, rows, V, out + 5, s);
  return e;
}

}  // namespace dspark
