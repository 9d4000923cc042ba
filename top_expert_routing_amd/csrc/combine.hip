// Gate-weighted combine back to token order, one wavefront per token.
//
// GRACE-MoE page, section 1: the combine exchange gathers expert outputs back
// to their tokens.  Each lane owns 8 consecutive features (one 16-byte load of
// bf16, two of fp32) and sums the k routed rows, then the shared rows, in fp32
// in that fixed order.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <bool BF16>
__global__ __launch_bounds__(kThreads) void combine_kernel(const void* __restrict__ h, const int* __restrict__ f2s,
                                                           const float* __restrict__ w, int T, int k, int S, int d,
                                                           void* __restrict__ y) {
  const int lane = lane_id();
  const int t = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const int groups8 = d / 8;
  for (int c8 = lane; c8 < groups8; c8 += kWave) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    for (int j = 0; j < k + S; ++j) {
      const int flat = j < k ? t * k + j : T * k + (j - k) * T + t;
      const int row = f2s[flat];
      const float wt = j < k ? w[static_cast<size_t>(t) * k + j] : 1.0f;
      if (BF16) {
        const uint4 v = reinterpret_cast<const uint4*>(h)[static_cast<size_t>(row) * groups8 + c8];
        const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += wt * __uint_as_float(p[q] << 16);
          acc[2 * q + 1] += wt * __uint_as_float(p[q] & 0xffff0000u);
        }
      } else {
        const float4* src = reinterpret_cast<const float4*>(h) + static_cast<size_t>(row) * (d / 4) + 2 * c8;
        const float4 a = src[0], b = src[1];
        const float v8[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += wt * v8[q];
      }
    }
    if (BF16) {
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      reinterpret_cast<uint4*>(y)[static_cast<size_t>(t) * groups8 + c8] = o;
    } else {
      float4* dst = reinterpret_cast<float4*>(y) + static_cast<size_t>(t) * (d / 4) + 2 * c8;
      dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

}  // namespace

hipError_t launch_combine(const void* h_sorted, const int* flat_to_sorted, const float* topk_w, int T, int k,
                          int n_shared, int d, int bf16, void* y, hipStream_t stream) {
  dim3 grid((T + kWaves - 1) / kWaves);
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(kThreads), 0, stream, h_sorted, flat_to_sorted, topk_w, T,
                       k, n_shared, d, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(kThreads), 0, stream, h_sorted, flat_to_sorted, topk_w, T,
                       k, n_shared, d, y);
  return hipGetLastError();
}

}  // namespace moe
