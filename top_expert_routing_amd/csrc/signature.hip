// Continuous request signature: for request r, layer l and expert e, the sum
// over the request's tokens of the full-E softmax probability of e.
//
// ELDR page, "Core idea / structure / operation": the paper compares its
// count x IDF signature against continuous alternatives such as the softmax
// gate probability; this is that alternative, read as the plain per-request
// sum without IDF.  NaN logits count as -inf and a token whose logits are all
// -inf adds nothing.
//
// One block per (request, layer).  The request's tokens go in chunks of 256:
// each wave takes a token at a time, holds its E <= 512 logits (8 per lane),
// and finds the maximum and the sum of exp(logit - max) with lane shuffles;
// the per-token maximum and 1/sum wait in LDS.  Then each thread adds, for its
// experts (e = tid, tid + 256), exp(logit - max) / sum of every token of the
// chunk in token order, so the result does not depend on scheduling.  All of
// it is double: the difference of two fp32 logits is exact there (in fp32 its
// rounding, up to |logit - max| * 2^-24, would pass straight into the
// probability), and the result is rounded to fp32 once.  The second pass
// re-reads the chunk's logits from L2.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunkTokens = 256;
constexpr int kPerLane = 8;                       // E <= 512 = 8 * 64
constexpr int kPerThread = 2;                     // E <= 512 = 2 * 256

__device__ __forceinline__ float finite_or_neg_inf(float v) { return v != v ? -__builtin_inff() : v; }

__global__ __launch_bounds__(kThreads) void prob_signature_kernel(const float* __restrict__ logits, int L, int T,
                                                                  int E, const int* __restrict__ offs,
                                                                  float* __restrict__ sig) {
  __shared__ float s_max[kChunkTokens];
  __shared__ double s_inv[kChunkTokens];          // 1 / sum, 0 for a token without a finite logit
  const int r = blockIdx.x, l = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int lo = min(max(offs[r], 0), T);
  const int hi = min(max(offs[r + 1], lo), T);
  const float* base = logits + static_cast<size_t>(l) * T * E;
  double acc[kPerThread] = {0.0, 0.0};

  for (int c0 = lo; c0 < hi; c0 += kChunkTokens) {
    const int c1 = min(hi, c0 + kChunkTokens);
    for (int t = c0 + wave; t < c1; t += kWaves) {
      const float* row = base + static_cast<size_t>(t) * E;
      float v[kPerLane];
      float m = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) {
        const int e = lane + kWave * i;
        v[i] = e < E ? finite_or_neg_inf(row[min(e, E - 1)]) : -__builtin_inff();
        m = fmaxf(m, v[i]);
      }
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
      double s = 0.0;
      if (m > -__builtin_inff()) {
#pragma unroll
        for (int i = 0; i < kPerLane; ++i)
          s += v[i] > -__builtin_inff() ? exp(static_cast<double>(v[i]) - static_cast<double>(m)) : 0.0;
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
      }
      if (lane == 0) {
        s_max[t - c0] = m;
        s_inv[t - c0] = m > -__builtin_inff() ? 1.0 / s : 0.0;
      }
    }
    __syncthreads();
    for (int t = c0; t < c1; ++t) {
      const double inv = s_inv[t - c0];
      if (inv == 0.0) continue;                   // the same for every thread
      const float m = s_max[t - c0];
      const float* row = base + static_cast<size_t>(t) * E;
#pragma unroll
      for (int q = 0; q < kPerThread; ++q) {
        const int e = threadIdx.x + kThreads * q;
        if (e < E) {
          const float x = finite_or_neg_inf(row[e]);
          if (x > -__builtin_inff()) acc[q] += exp(static_cast<double>(x) - static_cast<double>(m)) * inv;
        }
      }
    }
    __syncthreads();                              // s_max / s_inv are rewritten for the next chunk
  }
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int e = threadIdx.x + kThreads * q;
    if (e < E) sig[(static_cast<size_t>(r) * L + l) * E + e] = static_cast<float>(acc[q]);
  }
}

}  // namespace

hipError_t launch_prob_signature(const float* logits, int L, int T, int E, const int* req_offsets, int R,
                                 float* signature, hipStream_t stream) {
  hipLaunchKernelGGL(prob_signature_kernel, dim3(R, L), dim3(kThreads), 0, stream, logits, L, T, E, req_offsets,
                     signature);
  return hipGetLastError();
}

}  // namespace moe
