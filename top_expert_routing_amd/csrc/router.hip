// Router projection in front of the gate: one fp32 score per routed expert
// and token, logits[t][e] = sum_i x[t][i] * w_router[e][i].
//
// ELDR page, "Core idea / structure / operation": the gate is standard top-k
// gating over per-expert router scores of each token, left unchanged by the
// method.  The pages do not spell the router out; it is read here as the usual
// bias-free linear map of the token's hidden state (weights in the [out][in]
// layout of the expert matrices).
//
// bf16: one block of 16 waves per tile of 16*MF tokens x 16*NF experts.  The
// waves split the hidden dimension 16 ways, so a wave needs about one batch of
// loads (d = 2048: 128 values) and a block one memory round trip; each wave
// streams its slice of the tile's token rows and router rows straight into the
// v_mfma_f32_16x16x32_bf16 operands (a lane loads 16 bytes of one row per
// 32-wide K-step), all loads of a batch ahead of its first MFMA, and the
// slices' partial sums are added through LDS.  Small batches (decode) take
// 16 x 16 tiles, so even a few tokens spread over many CUs; large ones take
// 32 x 64 tiles, which read each token row once per 64 experts and each router
// row once per 32 tokens (the router matrix, at most 512 x d, stays in L2).
// Products of two bf16 values are exact in fp32, so the only rounding is the
// fp32 accumulation.
// fp32: one thread per (token, expert) dot product, 16-byte loads, fp32 FMA.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;        // 16 slices of the hidden dimension
constexpr int kF32Threads = 256;

template <int MF, int NF, int U>
__global__ __launch_bounds__(kThreads) void router_bf16(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ w, int T, int d, int E,
                                                        float* __restrict__ logits) {
  constexpr int KB = 32 * U;
  __shared__ f32x4 part[kWaves][MF * NF][kWave];

  const int t0 = blockIdx.x * 16 * MF, e0 = blockIdx.y * 16 * NF;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  const int l16 = lane & 15, q = lane >> 4;
  // this wave's slice of the hidden dimension, whole K-steps
  const int kq = (d + kWaves * 32 - 1) / (kWaves * 32) * 32;
  const int k0 = min(d, wave * kq), k1 = min(d, k0 + kq);

  // rows past T or E read the last valid row; their results are not stored
  const uint16_t* ap[MF];
  const uint16_t* bp[NF];
#pragma unroll
  for (int i = 0; i < MF; ++i) ap[i] = x + static_cast<size_t>(min(t0 + 16 * i + l16, T - 1)) * d + 8 * q;
#pragma unroll
  for (int j = 0; j < NF; ++j) bp[j] = w + static_cast<size_t>(min(e0 + 16 * j + l16, E - 1)) * d + 8 * q;

  f32x4 acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One batch of U K-steps from kc.  MASK: what lies at or past k1 is zeroed
  // (d and k1 are multiples of 8, so a lane's 8 values are all in or all out);
  // the load then reads the row's first 16 bytes instead.
  auto batch = [&](auto mask, int kc) {
    constexpr bool MASK = decltype(mask)::value;
    uint4 a[U][MF], b[U][NF];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = kc + 32 * u;
      const int ko = (!MASK || kk + 8 * q < k1) ? kk : -8 * q;
#pragma unroll
      for (int j = 0; j < NF; ++j) b[u][j] = *reinterpret_cast<const uint4*>(bp[j] + ko);
#pragma unroll
      for (int i = 0; i < MF; ++i) a[u][i] = *reinterpret_cast<const uint4*>(ap[i] + ko);
    }
    if constexpr (MASK) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (kc + 32 * u + 8 * q >= k1) {
#pragma unroll
          for (int j = 0; j < NF; ++j) b[u][j] = make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < MF; ++i) a[u][i] = make_uint4(0, 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // every load of the batch before its first MFMA
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b[u][j]),
                                                              __builtin_bit_cast(bf16x8, a[u][i]), acc[i][j], 0, 0, 0);
  };
  int kc = k0;
  for (; kc + KB <= k1; kc += KB) batch(std::false_type{}, kc);
  if (kc < k1) batch(std::true_type{}, kc);

  // Sum the slices.  The MFMA computes (router rows) x (token rows)^T: in each
  // 16x16 block a lane holds token 16 i + l16 and experts 16 j + 4q .. + 3.
  // Block p = i * NF + j is summed and stored by wave p % 16.
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) part[wave][i * NF + j][lane] = acc[i][j];
  __syncthreads();
#pragma unroll
  for (int p = 0; p < MF * NF; ++p) {
    if (p % kWaves != wave) continue;
    const int i = p / NF, j = p % NF;
    const int t = t0 + 16 * i + l16, e = e0 + 16 * j + 4 * q;
    if (t >= T || e >= E) continue;
    f32x4 s = part[0][p][lane];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) s += part[v][p][lane];
    float* out = logits + static_cast<size_t>(t) * E + e;
    if (e + 3 < E && ((static_cast<size_t>(t) * E + e) & 3) == 0) {
      *reinterpret_cast<f32x4*>(out) = s;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (e + c < E) out[c] = s[c];
    }
  }
}

// fp32: thread (token t, expert e) of a 16 x 16 tile; the dot product runs in
// index order with fp32 FMA, 4 values per load.
__global__ __launch_bounds__(kF32Threads) void router_f32(const float* __restrict__ x, const float* __restrict__ w,
                                                       int T, int d, int E, float* __restrict__ logits) {
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4), e = blockIdx.y * 16 + (threadIdx.x & 15);
  if (t >= T || e >= E) return;
  const float4* xr = reinterpret_cast<const float4*>(x + static_cast<size_t>(t) * d);
  const float4* wr = reinterpret_cast<const float4*>(w + static_cast<size_t>(e) * d);
  float s = 0.f;
  for (int i = 0; i < d / 4; ++i) {
    const float4 a = xr[i], b = wr[i];
    s = __builtin_fmaf(a.x, b.x, s);
    s = __builtin_fmaf(a.y, b.y, s);
    s = __builtin_fmaf(a.z, b.z, s);
    s = __builtin_fmaf(a.w, b.w, s);
  }
  logits[static_cast<size_t>(t) * E + e] = s;
}

}  // namespace

hipError_t launch_router(const void* x, const void* w_router, int T, int d, int E, int bf16, float* logits,
                         hipStream_t stream) {
  if (!bf16) {
    hipLaunchKernelGGL(router_f32, dim3((T + 15) / 16, (E + 15) / 16), dim3(kF32Threads), 0, stream,
                       static_cast<const float*>(x), static_cast<const float*>(w_router), T, d, E, logits);
    return hipGetLastError();
  }
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* wb = static_cast<const uint16_t*>(w_router);
  // 32 x 64 tiles once there are enough of them to give every CU one, 16 x 16 otherwise
  if (static_cast<long long>((T + 31) / 32) * ((E + 63) / 64) >= 256) {
    hipLaunchKernelGGL((router_bf16<2, 4, 2>), dim3((T + 31) / 32, (E + 63) / 64), dim3(kThreads), 0, stream, xb,
                       wb, T, d, E, logits);
  } else {
    hipLaunchKernelGGL((router_bf16<1, 1, 4>), dim3((T + 15) / 16, (E + 15) / 16), dim3(kThreads), 0, stream, xb,
                       wb, T, d, E, logits);
  }
  return hipGetLastError();
}

}  // namespace moe
