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


// One wave per (token, 512 features).  The k + S row indices are wave-uniform;
// rows are fetched 8 at a time so their loads overlap, then summed in order.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void combine_kernel(const void* __restrict__ h, const int* __restrict__ f2s,
                                                           const float* __restrict__ w, int T, int k, int S, int d,
                                                           int chunks, void* __restrict__ y) {
  const int lane = lane_id();
  const int wid = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (wid >= T * chunks) return;
  const int t = wid / chunks;
  const int c8 = (wid % chunks) * kWave + lane;     // 8-feature group of this lane
  const int groups8 = d / 8;
  const bool active = c8 < groups8;
  const int nrow = k + S;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
  for (int j0 = 0; j0 < nrow; j0 += 8) {
    int row[8];
    float wt[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = j0 + jj;
      row[jj] = 0;
      wt[jj] = 0.0f;
      if (j < nrow) {
        const int flat = j < k ? t * k + j : T * k + (j - k) * T + t;
        row[jj] = min(max(f2s[flat], 0), nrow * T - 1);   // a bad entry stays inside h
        wt[jj] = j < k ? w[static_cast<size_t>(t) * k + j] : 1.0f;
      }
    }
    if (BF16) {
      uint4 v[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        v[jj] = (active && j0 + jj < nrow)
                    ? reinterpret_cast<const uint4*>(h)[static_cast<size_t>(row[jj]) * groups8 + c8]
                    : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (j0 + jj >= nrow) break;
        const uint32_t p[4] = {v[jj].x, v[jj].y, v[jj].z, v[jj].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += wt[jj] * __uint_as_float(p[q] << 16);
          acc[2 * q + 1] += wt[jj] * __uint_as_float(p[q] & 0xffff0000u);
        }
      }
    } else {
      float4 va[8], vb[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        va[jj] = vb[jj] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (active && j0 + jj < nrow) {
          const float4* src = reinterpret_cast<const float4*>(h) + static_cast<size_t>(row[jj]) * (d / 4) + 2 * c8;
          va[jj] = src[0];
          vb[jj] = src[1];
        }
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (j0 + jj >= nrow) break;
        const float v8[8] = {va[jj].x, va[jj].y, va[jj].z, va[jj].w, vb[jj].x, vb[jj].y, vb[jj].z, vb[jj].w};
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += wt[jj] * v8[q];
      }
    }
  }
  if (!active) return;
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

}  // namespace

hipError_t launch_combine(const void* h_sorted, const int* flat_to_sorted, const float* topk_w, int T, int k,
                          int n_shared, int d, int bf16, void* y, hipStream_t stream) {
  const int chunks = (d / 8 + kWave - 1) / kWave;
  const long long waves = static_cast<long long>(T) * chunks;
  dim3 grid(static_cast<unsigned>((waves + kWaves - 1) / kWaves));
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(kThreads), 0, stream, h_sorted, flat_to_sorted, topk_w, T,
                       k, n_shared, d, chunks, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(kThreads), 0, stream, h_sorted, flat_to_sorted, topk_w, T,
                       k, n_shared, d, chunks, y);
  return hipGetLastError();
}

}  // namespace moe
