// Softmax top-k gate, one wavefront per token.
//
// ELDR page, "Core idea / structure / operation": the gate is standard top-k
// gating.  Each lane holds up to 8 of the row's logits as 64-bit keys
// (order-preserving bits of the value in the high word, the complement of the
// expert id in the low word), so the wave maximum is the largest logit with
// ties going to the lower id.  k rounds of a 6-step xor-shuffle maximum pick
// the experts in descending order; the owner lane retires the winner.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kMaxPerLane = 8;  // E <= 512
constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ uint64_t make_key(float v, int e) {
  if (v != v) v = -__builtin_inff();   // NaN ranks as -inf
  if (v == 0.0f) v = 0.0f;             // -0.0 and +0.0 tie
  uint32_t u = __float_as_uint(v);
  uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(0xffffffffu - static_cast<uint32_t>(e));
}

__device__ __forceinline__ float key_value(uint64_t key) {
  uint32_t ord = static_cast<uint32_t>(key >> 32);
  uint32_t u = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
  return __uint_as_float(u);
}

__device__ __forceinline__ int key_id(uint64_t key) {
  return static_cast<int>(0xffffffffu - static_cast<uint32_t>(key));
}

__global__ __launch_bounds__(kWave * kWavesPerBlock) void gate_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renormalize,
    int* __restrict__ topk_ids, float* __restrict__ topk_w) {
  const int lane = lane_id();
  const int t = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + static_cast<size_t>(t) * E;

  uint64_t keys[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    int e = lane + i * kWave;
    keys[i] = e < E ? make_key(row[e], e) : 0ull;   // 0 sorts below every real key
  }

  // chosen[i] holds slot (i*64 + lane) once it has been decided
  uint64_t chosen[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) chosen[i] = 0ull;

  for (int r = 0; r < k; ++r) {
    uint64_t best = keys[0];
#pragma unroll
    for (int i = 1; i < kMaxPerLane; ++i) best = keys[i] > best ? keys[i] : best;
    const uint64_t win = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      if (keys[i] == win) keys[i] = 0ull;           // ids are unique: one owner
      if ((r >> 6) == i && (r & 63) == lane) chosen[i] = win;
    }
  }

  // weights in double: renormalised softmax over the k chosen, or full softmax
  const uint64_t top = __shfl(chosen[0], 0, kWave);
  const double l0 = static_cast<double>(key_value(top));
  double z[kMaxPerLane];
  double part = 0.0;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int slot = i * kWave + lane;
    z[i] = 0.0;
    if (slot < k) {
      z[i] = exp(static_cast<double>(key_value(chosen[i])) - l0);
      if (renormalize) part += z[i];
    }
  }
  if (!renormalize) {
    // full softmax denominator over all E experts (max logit is slot 0's)
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      int e = lane + i * kWave;
      if (e < E) {
        float v = row[e];
        if (v != v) v = -__builtin_inff();
        part += exp(static_cast<double>(v) - l0);
      }
    }
  }
  const double denom = wave_sum(part);
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int slot = i * kWave + lane;
    if (slot < k) {
      topk_ids[static_cast<size_t>(t) * k + slot] = key_id(chosen[i]);
      topk_w[static_cast<size_t>(t) * k + slot] = static_cast<float>(z[i] / denom);
    }
  }
}

}  // namespace

hipError_t launch_gate(const float* logits, int T, int E, int k, int renormalize, int* topk_ids,
                       float* topk_w, hipStream_t stream) {
  dim3 grid((T + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(gate_kernel, grid, dim3(kWave * kWavesPerBlock), 0, stream, logits, T, E, k,
                     renormalize, topk_ids, topk_w);
  return hipGetLastError();
}

}  // namespace moe
