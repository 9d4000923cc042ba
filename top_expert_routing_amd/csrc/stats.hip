// Expert-activation statistics of a batch over a stack of layers.
//
// ELDR page, "What it solves": a decode step reads the union of distinct
// experts; "Core idea / structure / operation": per-request top-k activation
// counts reweighted by IDF form the request signature.  GRACE-MoE page,
// sections 3-4: co-activation (affinity) and per-expert load from recorded
// top-k selections.
//
// Small batches take a single-launch path (stats_small, below).  Otherwise two
// launches; all integer work is exact and order independent.
//   stats_count  grid (affinity row tiles + request chunks) x layers, two
//                block roles:
//                * affinity tile: LDS-privatised co-activation counts of every
//                  ordered slot pair of each token whose first expert falls in
//                  the tile's 16 rows, written out without global atomics;
//                  tile 0 also writes counts, union mask and union size.
//                * request chunk: LDS histograms of up to kReqChunk requests
//                  (tokens placed by binary search over the request offsets).
//   stats_idf    grid (64-expert chunks) x layers: document frequency over the
//                requests, idf = ln(R/df) in double (or the caller's idf), and
//                the signature.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kLdsInts = 16384;       // 64 KiB of LDS counters per block
constexpr int kAffRows = 16;          // affinity rows per tile
constexpr int kReqChunk = 32;         // requests per histogram block
constexpr int kIdsBuf = 4096;         // staged token ids per chunk

struct StatsGeom {
  int aff_tiles, rows_per_tile, req_chunks, rc;
};

StatsGeom geometry(int E, int R, bool want_aff, bool want_req) {
  StatsGeom g;
  g.rows_per_tile = want_aff ? (E < kAffRows ? E : kAffRows) : E;
  g.aff_tiles = want_aff ? (E + g.rows_per_tile - 1) / g.rows_per_tile : 1;
  g.rc = kLdsInts / E;
  if (g.rc > kReqChunk) g.rc = kReqChunk;
  g.req_chunks = want_req && R > 0 ? (R + g.rc - 1) / g.rc : 0;
  return g;
}

__global__ __launch_bounds__(kThreads) void stats_count(const int* __restrict__ ids, int L, int T, int k, int E,
                                                        StatsGeom geo, int* __restrict__ counts,
                                                        int* __restrict__ union_size,
                                                        uint8_t* __restrict__ union_mask, int* __restrict__ affinity,
                                                        const int* __restrict__ req_offsets, int R,
                                                        int* __restrict__ req_counts) {
  __shared__ int lds[kLdsInts];
  __shared__ int cnt[MOE_MAX_EXPERTS_DEV];
  __shared__ int offs[kReqChunk + 1];
  __shared__ int red[kThreads / kWave];
  __shared__ int idbuf[kIdsBuf];
  const int l = blockIdx.y;
  const int* lid = ids + static_cast<size_t>(l) * T * k;

  if (static_cast<int>(blockIdx.x) >= geo.aff_tiles) {
    // ---- request chunk: histograms of requests [r0, r0 + nr) ----
    const int r0 = (blockIdx.x - geo.aff_tiles) * geo.rc;
    const int nr = min(geo.rc, R - r0);
    for (int i = threadIdx.x; i < nr * E; i += kThreads) lds[i] = 0;
    for (int i = threadIdx.x; i <= nr; i += kThreads) offs[i] = max(0, min(req_offsets[r0 + i], T));
    __syncthreads();
    const int t_lo = offs[0], t_hi = max(offs[0], offs[nr]);
    // one thread per (token, slot): coalesced, independent loads
    for (int i = t_lo * k + threadIdx.x; i < t_hi * k; i += kThreads) {
      const int t = i / k;
      int lo = 0, hi = nr;                 // last r with offs[r] <= t
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offs[mid] <= t) lo = mid; else hi = mid;
      }
      if (t >= offs[lo + 1]) continue;     // not inside request lo (offsets not increasing)
      atomicAdd(&lds[lo * E + clamp_id(lid[i], E)], 1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nr * E; i += kThreads) {
      const int r = r0 + i / E, e = i % E;
      req_counts[(static_cast<size_t>(r) * L + l) * E + e] = lds[i];
    }
    return;
  }

  // ---- affinity tile: rows [a0, a0 + rows) of M^T M; tile 0 also counts ----
  // Token ids are staged through LDS in coalesced chunks; each thread then
  // walks the slot pairs of one token.
  const int a0 = blockIdx.x * geo.rows_per_tile;
  const int rows = min(geo.rows_per_tile, E - a0);
  const bool want_aff = affinity != nullptr;
  const bool tile0 = blockIdx.x == 0;
  if (want_aff)
    for (int i = threadIdx.x; i < rows * E; i += kThreads) lds[i] = 0;
  for (int e = threadIdx.x; e < E; e += kThreads) cnt[e] = 0;
  const int tb = kIdsBuf / k;            // tokens per staged chunk (k <= 512)
  for (int t0 = 0; t0 < T; t0 += tb) {
    const int nt = min(tb, T - t0);
    __syncthreads();
    for (int i = threadIdx.x; i < nt * k; i += kThreads)
      idbuf[i] = clamp_id(lid[static_cast<size_t>(t0) * k + i], E);
    __syncthreads();
    for (int tt = threadIdx.x; tt < nt; tt += kThreads) {
      const int* row = idbuf + tt * k;
      for (int j1 = 0; j1 < k; ++j1) {
        const int a = row[j1];
        if (tile0) atomicAdd(&cnt[a], 1);
        if (!want_aff || a < a0 || a >= a0 + rows) continue;
        int* dst = lds + (a - a0) * E;
        for (int j2 = 0; j2 < k; ++j2) atomicAdd(&dst[row[j2]], 1);
      }
    }
  }
  __syncthreads();
  if (want_aff) {
    int* dst = affinity + (static_cast<size_t>(l) * E + a0) * E;
    for (int i = threadIdx.x; i < rows * E; i += kThreads) dst[i] = lds[i];
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

// One block of 16 waves per (64-expert chunk, layer): lanes own an expert, the
// waves split the requests; loads are issued kBatch at a time so a batch of
// 128 requests costs one memory latency.
constexpr int kIdfThreads = 1024;
constexpr int kBatch = 8;

__global__ __launch_bounds__(kIdfThreads) void stats_idf(int L, int E, int R, const int* __restrict__ req_counts,
                                                         const float* __restrict__ idf_in,
                                                         float* __restrict__ signature) {
  constexpr int kW = kIdfThreads / kWave;
  __shared__ int dfp[kW][kWave];
  __shared__ double idf[kWave];
  const int l = blockIdx.y;
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int e = blockIdx.x * kWave + lane;
  const bool ok = e < E;
  const int ec = ok ? e : 0;
  const size_t rstride = static_cast<size_t>(L) * E;
  const int* base = req_counts + static_cast<size_t>(l) * E + ec;
  int df = 0;
  if (!idf_in) {
    for (int r0 = w; r0 < R; r0 += kW * kBatch) {
      int v[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int r = r0 + b * kW;
        v[b] = (ok && r < R) ? base[static_cast<size_t>(r) * rstride] : 0;
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) df += v[b] > 0;
    }
  }
  dfp[w][lane] = df;
  __syncthreads();
  if (w == 0 && ok) {
    if (idf_in) {
      idf[lane] = static_cast<double>(idf_in[static_cast<size_t>(l) * E + e]);
    } else {
      int d = 0;
      for (int i = 0; i < kW; ++i) d += dfp[i][lane];
      idf[lane] = d > 0 ? log(static_cast<double>(R) / static_cast<double>(d)) : 0.0;
    }
  }
  __syncthreads();
  if (!ok) return;
  const double f = idf[lane];
  float* sbase = signature + static_cast<size_t>(l) * E + e;
  for (int r0 = w; r0 < R; r0 += kW * kBatch) {
    int v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int r = r0 + b * kW;
      v[b] = r < R ? base[static_cast<size_t>(r) * rstride] : 0;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int r = r0 + b * kW;
      if (r < R) sbase[static_cast<size_t>(r) * rstride] = static_cast<float>(static_cast<double>(v[b]) * f);
    }
  }
}

// ---- small batches: everything for one layer in one 1024-thread block ---------
// When the affinity matrix, the request histograms and the request offsets fit
// in 56 KiB of LDS, one block per layer computes counts, union, affinity,
// request counts, idf and signature in a single launch (decode-sized batches:
// the two-launch path would pay a second launch and a global round trip).
constexpr int kSmallThreads = 1024;
constexpr int kSmallLds = 14336;     // ints shared by affinity, request counts, offsets

bool small_fits(int E, int R, bool want_aff, bool want_req, int T, int k) {
  const long long need = (want_aff ? 1LL * E * E : 0) + (want_req ? 1LL * R * E + R + 1 : 0);
  return need <= kSmallLds && 1LL * T * k <= (1LL << 20);
}

__global__ __launch_bounds__(kSmallThreads) void stats_small(const int* __restrict__ ids, int L, int T, int k,
                                                             int E, int* __restrict__ counts,
                                                             int* __restrict__ union_size,
                                                             uint8_t* __restrict__ union_mask,
                                                             int* __restrict__ affinity,
                                                             const int* __restrict__ req_offsets, int R,
                                                             const float* __restrict__ idf_in,
                                                             int* __restrict__ req_counts,
                                                             float* __restrict__ signature) {
  __shared__ int lds[kSmallLds];
  __shared__ int cnt[MOE_MAX_EXPERTS_DEV];
  __shared__ double idf[MOE_MAX_EXPERTS_DEV];
  __shared__ int red[kSmallThreads / kWave];
  const int l = blockIdx.x;
  const int tid = threadIdx.x;
  const bool want_aff = affinity != nullptr;
  const bool want_req = req_offsets != nullptr && R > 0 && (req_counts != nullptr || signature != nullptr);
  int* aff = lds;
  int* req = lds + (want_aff ? E * E : 0);
  int* offs = req + (want_req ? R * E : 0);
  const int used = (want_aff ? E * E : 0) + (want_req ? R * E : 0);
  for (int i = tid; i < used; i += kSmallThreads) lds[i] = 0;
  for (int e = tid; e < E; e += kSmallThreads) cnt[e] = 0;
  if (want_req)
    for (int i = tid; i <= R; i += kSmallThreads) offs[i] = max(0, min(req_offsets[i], T));
  __syncthreads();
  const int* lid = ids + static_cast<size_t>(l) * T * k;
  for (int t = tid; t < T; t += kSmallThreads) {
    int r = -1;
    if (want_req && t >= offs[0] && t < offs[R]) {
      int lo = 0, hi = R;                   // last r with offs[r] <= t
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offs[mid] <= t) lo = mid; else hi = mid;
      }
      if (t < offs[lo + 1]) r = lo;
    }
    const int* row = lid + static_cast<size_t>(t) * k;
    for (int j0 = 0; j0 < k; j0 += 8) {
      int idv[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) idv[jj] = j0 + jj < k ? clamp_id(row[j0 + jj], E) : -1;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int a = idv[jj];
        if (a < 0) break;
        atomicAdd(&cnt[a], 1);
        if (r >= 0) atomicAdd(&req[r * E + a], 1);
        if (want_aff)
          for (int j2 = 0; j2 < k; ++j2) atomicAdd(&aff[a * E + clamp_id(row[j2], E)], 1);
      }
    }
  }
  __syncthreads();
  int nz = 0;
  for (int e = tid; e < E; e += kSmallThreads) {
    const int c = cnt[e];
    counts[static_cast<size_t>(l) * E + e] = c;
    if (union_mask) union_mask[static_cast<size_t>(l) * E + e] = c > 0 ? 1 : 0;
    nz += c > 0 ? 1 : 0;
    if (want_req && signature) {
      if (idf_in) {
        idf[e] = static_cast<double>(idf_in[static_cast<size_t>(l) * E + e]);
      } else {
        int df = 0;
        for (int rr = 0; rr < R; ++rr) df += req[rr * E + e] > 0;
        idf[e] = df > 0 ? log(static_cast<double>(R) / static_cast<double>(df)) : 0.0;
      }
    }
  }
  nz = wave_sum(nz);
  if (lane_id() == 0) red[tid >> 6] = nz;
  if (want_aff) {
    int* dst = affinity + static_cast<size_t>(l) * E * E;
    for (int i = tid; i < E * E; i += kSmallThreads) dst[i] = aff[i];
  }
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int w = 0; w < kSmallThreads / kWave; ++w) s += red[w];
    union_size[l] = s;
  }
  if (!want_req) return;
  for (int i = tid; i < R * E; i += kSmallThreads) {
    const int rr = i / E, e = i % E;
    const size_t at = (static_cast<size_t>(rr) * L + l) * E + e;
    if (req_counts) req_counts[at] = req[i];
    if (signature) signature[at] = static_cast<float>(static_cast<double>(req[i]) * idf[e]);
  }
}

}  // namespace

size_t stats_workspace_bytes(int L, int T, int k, int E, int R) {
  (void)T;
  (void)k;
  // request counts go through the workspace when the caller wants only the
  // signature
  return static_cast<size_t>(((static_cast<long long>(R) * L * E * 4) + 255) / 256 * 256 + 256);
}

hipError_t launch_stats(const StatsArgs& a, void* workspace, hipStream_t stream) {
  if (a.L == 0) return hipSuccess;
  const bool want_req = a.req_offsets && a.R > 0 && (a.req_counts || a.signature);
  if (small_fits(a.E, a.R, a.affinity != nullptr, want_req, a.T, a.k)) {
    hipLaunchKernelGGL(stats_small, dim3(a.L), dim3(kSmallThreads), 0, stream, a.topk_ids, a.L, a.T, a.k, a.E,
                       a.counts, a.union_size, a.union_mask, a.affinity, want_req ? a.req_offsets : nullptr,
                       want_req ? a.R : 0, a.idf, a.req_counts, a.signature);
    return hipGetLastError();
  }
  const StatsGeom geo = geometry(a.E, a.R, a.affinity != nullptr, want_req);
  int* rc = a.req_counts ? a.req_counts : static_cast<int*>(workspace);
  hipLaunchKernelGGL(stats_count, dim3(geo.aff_tiles + geo.req_chunks, a.L), dim3(kThreads), 0, stream, a.topk_ids,
                     a.L, a.T, a.k, a.E, geo, a.counts, a.union_size, a.union_mask, a.affinity, a.req_offsets, a.R,
                     rc);
  if (want_req && a.signature)
    hipLaunchKernelGGL(stats_idf, dim3((a.E + kWave - 1) / kWave, a.L), dim3(kIdfThreads), 0, stream, a.L, a.E, a.R,
                       static_cast<const int*>(rc), a.idf, a.signature);
  return hipGetLastError();
}

}  // namespace moe
