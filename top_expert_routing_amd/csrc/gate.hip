// Softmax top-k gate, one wavefront per token.
//
// ELDR page, "Core idea / structure / operation": the gate is standard top-k
// gating.  Each lane holds P = ceil(E/64) of the row's logits (expert
// e = 64 i + lane in slot i) as order-preserving 32-bit keys.  k rounds pick
// the experts in descending order: the wave maximum of the keys comes from
// four DPP steps inside each 16-lane row and four lane reads, and the winner
// among equal keys (the lowest expert id) from one ballot per slot; the winning
// slot is retired.  No LDS traffic and no shuffles through the LDS crossbar.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kWavesPerBlock = 4;

// Monotone map of a logit to uint32 (NaN ranks as -inf, -0.0 ties +0.0).
// 0 is below every key it returns, so it marks retired and empty slots.
__device__ __forceinline__ uint32_t ord_key(float v) {
  if (v != v) v = -__builtin_inff();
  if (v == 0.0f) v = 0.0f;
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t ord) {
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
  return __uint_as_float(u);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, 0xf, 0xf,
                                                           false));
}

// Maximum over the 64 lanes (all lanes active), returned wave-uniform.
__device__ __forceinline__ uint32_t wave_max_key(uint32_t v) {
  v = max(v, dpp<0xb1>(v));    // quad_perm [1,0,3,2]: lane ^ 1
  v = max(v, dpp<0x4e>(v));    // quad_perm [2,3,0,1]: lane ^ 2
  v = max(v, dpp<0x141>(v));   // row_half_mirror: 8-lane halves
  v = max(v, dpp<0x140>(v));   // row_mirror: 16-lane rows
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

// The gate of token t on one wave (every lane active).  With `hist` (LDS),
// each chosen expert's counter is also incremented once per slot.
template <int P>
__device__ __forceinline__ void gate_token(const float* __restrict__ logits, int t, int E, int k, int renormalize,
                                           int* __restrict__ topk_ids, float* __restrict__ topk_w, int* hist) {
  const int lane = lane_id();
  const float* row = logits + static_cast<size_t>(t) * E;

  uint32_t key[P], orig[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int e = lane + i * kWave;
    orig[i] = e < E ? ord_key(row[e]) : 0u;
    key[i] = orig[i];
  }

  // round r is kept by lane r % 64 in slot r / 64
  uint32_t cval[P];
  int cid[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    cval[i] = 0u;
    cid[i] = 0;
  }
  uint32_t top = 0u;
  for (int r = 0; r < k; ++r) {
    uint32_t best = key[0];
#pragma unroll
    for (int i = 1; i < P; ++i) best = max(best, key[i]);
    const uint32_t win = wave_max_key(best);
    if (r == 0) top = win;
    int wi = 0, wl = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const uint64_t m = __ballot(key[i] == win);
      if (m) {
        wi = i;
        wl = __ffsll(static_cast<unsigned long long>(m)) - 1;
        break;
      }
    }
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (i == wi && lane == wl) key[i] = 0u;
      if (r == i * kWave + lane) {
        cval[i] = win;
        cid[i] = wi * kWave + wl;
      }
    }
  }

  // weights in double: renormalised softmax over the k chosen, or full softmax
  const double l0 = static_cast<double>(key_value(top));
  double z[P];
  double part = 0.0;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int slot = i * kWave + lane;
    z[i] = 0.0;
    if (slot < k) {
      z[i] = exp(static_cast<double>(key_value(cval[i])) - l0);
      if (renormalize) part += z[i];
    }
  }
  if (!renormalize) {
    // full softmax denominator over all E experts (the maximum is slot 0's)
#pragma unroll
    for (int i = 0; i < P; ++i)
      if (lane + i * kWave < E) part += exp(static_cast<double>(key_value(orig[i])) - l0);
  }
  const double denom = wave_sum(part);
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int slot = i * kWave + lane;
    if (slot < k) {
      topk_ids[static_cast<size_t>(t) * k + slot] = cid[i];
      topk_w[static_cast<size_t>(t) * k + slot] = static_cast<float>(z[i] / denom);
      if (hist) atomicAdd(hist + cid[i], 1);
    }
  }
}

template <int P>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void gate_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renormalize,
    int* __restrict__ topk_ids, float* __restrict__ topk_w) {
  const int t = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;    // whole waves leave: every lane of a live wave is active
  gate_token<P>(logits, t, E, k, renormalize, topk_ids, topk_w, nullptr);
}

// Gate plus KV-block recording (ELDR page, "Core idea / structure /
// operation": expert activations recorded per KV block during prefill).  One
// block per KV block of `bt` tokens, min(bt, 16) waves taking its tokens in
// turn; the block's expert histogram lives in LDS and is written out whole
// (zeros included) as row (b, layer) of block_counts [nblocks][L][E], so no
// global atomics and no clearing pass are needed, and the counts are exact.
constexpr int kRecordMaxWaves = 16;

template <int P>
__global__ __launch_bounds__(kWave * kRecordMaxWaves) void gate_record_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renormalize, int* __restrict__ topk_ids,
    float* __restrict__ topk_w, int bt, int layer, int L, int* __restrict__ block_counts) {
  __shared__ int hist[P * kWave];
  const int nw = blockDim.x >> 6, w = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const long long t0 = static_cast<long long>(blockIdx.x) * bt;
  const long long t1 = min(static_cast<long long>(T), t0 + bt);
  for (long long t = t0 + w; t < t1; t += nw)
    gate_token<P>(logits, static_cast<int>(t), E, k, renormalize, topk_ids, topk_w, hist);
  __syncthreads();
  int* out = block_counts + (static_cast<size_t>(blockIdx.x) * L + layer) * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) out[e] = hist[e];
}

}  // namespace

hipError_t launch_gate(const float* logits, int T, int E, int k, int renormalize, int* topk_ids,
                       float* topk_w, hipStream_t stream) {
  dim3 grid((T + kWavesPerBlock - 1) / kWavesPerBlock), block(kWave * kWavesPerBlock);
  if (E <= 64)
    hipLaunchKernelGGL(gate_kernel<1>, grid, block, 0, stream, logits, T, E, k, renormalize, topk_ids, topk_w);
  else if (E <= 128)
    hipLaunchKernelGGL(gate_kernel<2>, grid, block, 0, stream, logits, T, E, k, renormalize, topk_ids, topk_w);
  else if (E <= 256)
    hipLaunchKernelGGL(gate_kernel<4>, grid, block, 0, stream, logits, T, E, k, renormalize, topk_ids, topk_w);
  else
    hipLaunchKernelGGL(gate_kernel<8>, grid, block, 0, stream, logits, T, E, k, renormalize, topk_ids, topk_w);
  return hipGetLastError();
}

hipError_t launch_gate_record(const float* logits, int T, int E, int k, int renormalize, int* topk_ids,
                              float* topk_w, int block_tokens, int layer, int L, int* block_counts,
                              hipStream_t stream) {
  const int nblocks = static_cast<int>((static_cast<long long>(T) + block_tokens - 1) / block_tokens);
  dim3 grid(nblocks), block(kWave * (block_tokens < kRecordMaxWaves ? block_tokens : kRecordMaxWaves));
  if (E <= 64)
    hipLaunchKernelGGL(gate_record_kernel<1>, grid, block, 0, stream, logits, T, E, k, renormalize, topk_ids, topk_w,
                       block_tokens, layer, L, block_counts);
  else if (E <= 128)
    hipLaunchKernelGGL(gate_record_kernel<2>, grid, block, 0, stream, logits, T, E, k, renormalize, topk_ids, topk_w,
                       block_tokens, layer, L, block_counts);
  else if (E <= 256)
    hipLaunchKernelGGL(gate_record_kernel<4>, grid, block, 0, stream, logits, T, E, k, renormalize, topk_ids, topk_w,
                       block_tokens, layer, L, block_counts);
  else
    hipLaunchKernelGGL(gate_record_kernel<8>, grid, block, 0, stream, logits, T, E, k, renormalize, topk_ids, topk_w,
                       block_tokens, layer, L, block_counts);
  return hipGetLastError();
}

}  // namespace moe
