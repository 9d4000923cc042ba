// Expert-activation statistics of a batch over a stack of layers.
//
// ELDR page, "What it solves": a decode step reads the union of distinct
// experts; "Core idea / structure / operation": per-request top-k activation
// counts reweighted by IDF form the request signature.  GRACE-MoE page,
// sections 3-4: co-activation (affinity) and per-expert load from recorded
// top-k selections.
//
// Three launches, all integer work exact and order independent:
//   stats_layer   one block per (layer, tile of affinity rows): LDS-privatised
//                 co-activation counts (every ordered slot pair of a token),
//                 written out without global atomics; tile 0 also writes the
//                 counts, union mask and union size.
//   stats_request one block per (request, layer): LDS histogram of the
//                 request's tokens.
//   stats_idf     one block per layer: document frequency over the requests,
//                 idf = ln(R/df) in double (or the caller's idf), signature.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kAffLdsInts = 16384;   // 64 KiB of affinity counters per block

__global__ __launch_bounds__(kThreads) void stats_layer(const int* __restrict__ ids, int T, int k, int E,
                                                        int rows_per_tile, int* __restrict__ counts,
                                                        int* __restrict__ union_size, uint8_t* __restrict__ union_mask,
                                                        int* __restrict__ affinity) {
  __shared__ int aff[kAffLdsInts];
  __shared__ int cnt[MOE_MAX_EXPERTS_DEV];
  __shared__ int red[kThreads / kWave];
  const int l = blockIdx.y;
  const int r0 = blockIdx.x * rows_per_tile;
  const int rows = min(rows_per_tile, E - r0);
  const bool want_aff = affinity != nullptr;
  const bool tile0 = blockIdx.x == 0;
  if (want_aff)
    for (int i = threadIdx.x; i < rows * E; i += kThreads) aff[i] = 0;
  for (int e = threadIdx.x; e < E; e += kThreads) cnt[e] = 0;
  __syncthreads();
  const int* lid = ids + static_cast<size_t>(l) * T * k;
  // one token per thread; every ordered slot pair (a, b) with a in this tile
  for (int t = threadIdx.x; t < T; t += kThreads) {
    const int* row = lid + static_cast<size_t>(t) * k;
    for (int j1 = 0; j1 < k; ++j1) {
      const int a = clamp_id(row[j1], E);
      if (tile0) atomicAdd(&cnt[a], 1);
      if (!want_aff || a < r0 || a >= r0 + rows) continue;
      for (int j2 = 0; j2 < k; ++j2) atomicAdd(&aff[(a - r0) * E + clamp_id(row[j2], E)], 1);
    }
  }
  __syncthreads();
  if (want_aff) {
    int* dst = affinity + (static_cast<size_t>(l) * E + r0) * E;
    for (int i = threadIdx.x; i < rows * E; i += kThreads) dst[i] = aff[i];
  }
  if (!tile0) return;
  int nz = 0;
  for (int e = threadIdx.x; e < E; e += kThreads) {
    const int c = cnt[e];
    counts[static_cast<size_t>(l) * E + e] = c;
    if (union_mask) union_mask[static_cast<size_t>(l) * E + e] = c > 0 ? 1 : 0;
    nz += c > 0 ? 1 : 0;
  }
  nz = wave_sum(nz);
  if (lane_id() == 0) red[threadIdx.x >> 6] = nz;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int w = 0; w < kThreads / kWave; ++w) s += red[w];
    union_size[l] = s;
  }
}

__global__ __launch_bounds__(kThreads) void stats_request(const int* __restrict__ ids, int L, int T, int k, int E,
                                                          const int* __restrict__ req_offsets,
                                                          int* __restrict__ req_counts) {
  __shared__ int cnt[MOE_MAX_EXPERTS_DEV];
  const int r = blockIdx.x, l = blockIdx.y;
  for (int e = threadIdx.x; e < E; e += kThreads) cnt[e] = 0;
  __syncthreads();
  int lo = req_offsets[r], hi = req_offsets[r + 1];
  lo = max(0, min(lo, T));
  hi = max(lo, min(hi, T));
  const int* lid = ids + static_cast<size_t>(l) * T * k;
  for (int i = lo * k + threadIdx.x; i < hi * k; i += kThreads) atomicAdd(&cnt[clamp_id(lid[i], E)], 1);
  __syncthreads();
  int* dst = req_counts + (static_cast<size_t>(r) * L + l) * E;
  for (int e = threadIdx.x; e < E; e += kThreads) dst[e] = cnt[e];
}

__global__ __launch_bounds__(kThreads) void stats_idf(int L, int E, int R, const int* __restrict__ req_counts,
                                                      const float* __restrict__ idf_in, float* __restrict__ signature) {
  __shared__ double idf[MOE_MAX_EXPERTS_DEV];
  const int l = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kThreads) {
    if (idf_in) {
      idf[e] = static_cast<double>(idf_in[static_cast<size_t>(l) * E + e]);
    } else {
      int df = 0;
      for (int r = 0; r < R; ++r) df += req_counts[(static_cast<size_t>(r) * L + l) * E + e] > 0 ? 1 : 0;
      idf[e] = df > 0 ? log(static_cast<double>(R) / static_cast<double>(df)) : 0.0;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < R * E; i += kThreads) {
    const int r = i / E, e = i % E;
    const size_t at = (static_cast<size_t>(r) * L + l) * E + e;
    signature[at] = static_cast<float>(static_cast<double>(req_counts[at]) * idf[e]);
  }
}

}  // namespace

size_t stats_workspace_bytes(int L, int T, int k, int E, int R) {
  (void)T;
  (void)k;
  // per-request counts are needed for the signature even when the caller does
  // not ask for them
  return static_cast<size_t>(((static_cast<long long>(R) * L * E * 4) + 255) / 256 * 256 + 256);
}

hipError_t launch_stats(const StatsArgs& a, void* workspace, hipStream_t stream) {
  if (a.L == 0) return hipSuccess;
  int rows_per_tile = a.E;
  if (a.affinity) {
    rows_per_tile = kAffLdsInts / a.E;
    if (rows_per_tile > a.E) rows_per_tile = a.E;
  }
  const int tiles = a.affinity ? (a.E + rows_per_tile - 1) / rows_per_tile : 1;
  hipLaunchKernelGGL(stats_layer, dim3(tiles, a.L), dim3(kThreads), 0, stream, a.topk_ids, a.T, a.k, a.E,
                     rows_per_tile, a.counts, a.union_size, a.union_mask, a.affinity);
  if (a.req_offsets && a.R > 0 && (a.req_counts || a.signature)) {
    int* rc = a.req_counts ? a.req_counts : static_cast<int*>(workspace);
    hipLaunchKernelGGL(stats_request, dim3(a.R, a.L), dim3(kThreads), 0, stream, a.topk_ids, a.L, a.T, a.k, a.E,
                       a.req_offsets, rc);
    if (a.signature)
      hipLaunchKernelGGL(stats_idf, dim3(a.L), dim3(kThreads), 0, stream, a.L, a.E, a.R,
                         static_cast<const int*>(rc), a.idf, a.signature);
  }
  return hipGetLastError();
}

}  // namespace moe
