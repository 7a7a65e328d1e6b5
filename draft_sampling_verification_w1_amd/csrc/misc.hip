// misc.hip -- W2 packing (once per model) and the confidence head.
#include "device_common.h"
#include "kernels.h"

namespace dspark {

namespace {

// Packed bf16 W2: tile t of 32 tokens, step s of 16 rank indices, lane l:
// the 8 values W2[128*(l/32) + 8*s + e][32*t + pi(l%32)], e = 0..7, where
// pi(m) = 16*((m>>2)&1) + 4*(m>>3) + (m&3) undoes the MFMA 32x32 output row
// order so that each lane ends up with 16 consecutive tokens.
__global__ __launch_bounds__(256) void k_pack_w2_bf16(int V, int ntiles, const uint16_t* W2,
                                                      u32x4* out) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= (int64_t)ntiles * kSteps * 64) return;
  const int l = (int)(g & 63);
  const int s = (int)((g >> 6) % kSteps);
  const int t = (int)(g / (64 * kSteps));
  const int m = l & 31;
  const int v = t * kTile + 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
  const int k0 = 128 * (l >> 5) + 8 * s;
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = v < V ? W2[(int64_t)(k0 + 2 * e) * V + v] : 0u;
    const uint32_t hi = v < V ? W2[(int64_t)(k0 + 2 * e + 1) * V + v] : 0u;
    w[e] = lo | (hi << 16);
  }
  out[g] = (u32x4){w[0], w[1], w[2], w[3]};
}

// Largest |W2[i][v]| over the rank and the 32 tokens of each tile: the
// per-tile factor of the contraction's error bound that the split passes use
// to bracket their binary32 scores.  Read from the packed tiles (contiguous:
// 16 KB bf16, 32 KB binary32), whose entries for tokens at or beyond V are
// zeros and never raise it; one workgroup per tile, after the packing kernel.
template <bool BF16>
__global__ __launch_bounds__(256) void k_tile_absmax(const u32x4* W2p, float* tmax) {
  constexpr int kChunks = BF16 ? kSteps * 64 : kTile * kRank / 4;  // 16-byte chunks per tile
  __shared__ float part[4];
  const int t = blockIdx.x;
  const u32x4* tile = W2p + (int64_t)t * kChunks;
  float m = 0.f;
#pragma unroll
  for (int c = threadIdx.x; c < kChunks; c += 256) {
    const u32x4 q = tile[c];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (BF16) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[e])), fabsf(bf16_hi(w[e]))));
      else m = fmaxf(m, fabsf(__uint_as_float(w[e])));
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) tmax[t] = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
}

// Transposed f32 W2: out[v][i] = W2[i][v], zero rows for v >= V.
__global__ __launch_bounds__(256) void k_pack_w2_f32(int V, int vpad, const float* W2, float* out) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= (int64_t)vpad * kRank) return;
  const int i = (int)(g % kRank);
  const int v = (int)(g / kRank);
  out[g] = v < V ? W2[(int64_t)i * V + v] : 0.0f;
}

// Confidence head with per-position temperature (summary page §3.2.1):
// c = sigmoid((w . [h_k; W1[x_{k-1}]]) / T_k), one wave per row, binary64 sums.
// VEC: h rows and w 16-byte aligned (H a multiple of 8), 8 entries per load.
template <typename E, bool VEC>
__global__ __launch_bounds__(256) void k_confidence(int R, int gamma, int V, int H,
                                                    const uint16_t* h, const float* w,
                                                    const float* temps, const E* W1,
                                                    const int32_t* anchors, const int32_t* tokens,
                                                    float* c) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R * gamma) return;
  const int r = row / gamma;
  const int k = row - r * gamma + 1;
  int x = (k == 1) ? anchors[r] : tokens[(int64_t)r * gamma + (k - 2)];
  x = min(max(x, 0), V - 1);
  const uint16_t* hr = h + (int64_t)row * H;
  double s = 0.0;
  if constexpr (VEC) {
    for (int i = 8 * lane; i < H; i += 512) {
      const u32x4 hv = *reinterpret_cast<const u32x4*>(hr + i);
      const f32x4 wa = *reinterpret_cast<const f32x4*>(w + i);
      const f32x4 wb = *reinterpret_cast<const f32x4*>(w + i + 4);
      const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
      const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t bits = (e & 1) ? (hw[e >> 1] & 0xFFFF0000u) : (hw[e >> 1] << 16);
        s += (double)wv[e] * (double)__uint_as_float(bits);
      }
    }
  } else {
    for (int i = lane; i < H; i += 64) s += (double)w[i] * (double)bf16_at(hr, i);
  }
  for (int j = lane; j < kRank; j += 64)
    s += (double)w[H + j] * (double)elem_at(W1, (int64_t)x * kRank + j);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) c[row] = (float)(1.0 / (1.0 + exp(-s / (double)temps[k - 1])));
}

// log p^d = z - lse per drafted row, in place over the logits the draft
// stored: the difference in binary64, rounded once to binary32.
__global__ __launch_bounds__(256) void k_logpd(int V, const double* lse, float* zl) {
  const int64_t row = blockIdx.y;
  const double l = lse[row];
  float* p = zl + row * (int64_t)V;
  for (int v = blockIdx.x * 256 + threadIdx.x; v < V; v += gridDim.x * 256)
    p[v] = (float)((double)p[v] - l);
}

}  // namespace

hipError_t launch_logpd(int rows, int V, const double* lse, float* zl, hipStream_t stream) {
  TimingScope timing("logpd", stream);
  const int chunks = (V + 4095) / 4096;
  hipLaunchKernelGGL(k_logpd, dim3(chunks, rows), dim3(256), 0, stream, V, lse, zl);
  return hipGetLastError();
}

hipError_t launch_pack_w2(bool bf16, int V, const void* W2, void* W2p, hipStream_t stream) {
  TimingScope timing("pack_w2", stream);
  const int ntiles = (V + kTile - 1) / kTile;
  float* tmax = w2_tile_absmax(W2p, bf16, ntiles);
  if (bf16) {
    const int64_t n = (int64_t)ntiles * kSteps * 64;
    hipLaunchKernelGGL(k_pack_w2_bf16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, V,
                       ntiles, (const uint16_t*)W2, (u32x4*)W2p);
    hipLaunchKernelGGL(k_tile_absmax<true>, dim3(ntiles), dim3(256), 0, stream,
                       (const u32x4*)W2p, tmax);
  } else {
    const int64_t n = (int64_t)ntiles * kTile * kRank;
    hipLaunchKernelGGL(k_pack_w2_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, V,
                       ntiles * kTile, (const float*)W2, (float*)W2p);
    hipLaunchKernelGGL(k_tile_absmax<false>, dim3(ntiles), dim3(256), 0, stream,
                       (const u32x4*)W2p, tmax);
  }
  return hipGetLastError();
}

hipError_t launch_confidence(bool w1_bf16, int R, int gamma, int V, int H, const uint16_t* h,
                             const float* w, const float* temps, const void* W1,
                             const int32_t* anchors, const int32_t* tokens, float* c,
                             hipStream_t stream) {
  TimingScope timing("confidence", stream);
  const int rows = R * gamma;
  const dim3 grid((rows + 3) / 4);
  const bool vec = H % 8 == 0 && ((uintptr_t)h & 15u) == 0 && ((uintptr_t)w & 15u) == 0;
  if (w1_bf16 && vec)
    hipLaunchKernelGGL((k_confidence<uint16_t, true>), grid, dim3(256), 0, stream, R, gamma, V, H,
                       h, w, temps, (const uint16_t*)W1, anchors, tokens, c);
  else if (w1_bf16)
    hipLaunchKernelGGL((k_confidence<uint16_t, false>), grid, dim3(256), 0, stream, R, gamma, V, H,
                       h, w, temps, (const uint16_t*)W1, anchors, tokens, c);
  else if (vec)
    hipLaunchKernelGGL((k_confidence<float, true>), grid, dim3(256), 0, stream, R, gamma, V, H, h,
                       w, temps, (const float*)W1, anchors, tokens, c);
  else
    hipLaunchKernelGGL((k_confidence<float, false>), grid, dim3(256), 0, stream, R, gamma, V, H, h,
                       w, temps, (const float*)W1, anchors, tokens, c);
  return hipGetLastError();
}

}  // namespace dspark
