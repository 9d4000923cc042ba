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
//   stats_count  grid (affinity row tiles x token splits + request chunks) x
//                layers, two block roles:
//                * affinity tile: LDS-privatised co-activation counts of every
//                  ordered slot pair of each token of the split whose first
//                  expert falls in the tile's rows (16, or as many as 32 KiB
//                  of counters hold when the ids are split); tile 0 also
//                  counts.
//                  With one split the block writes the outputs; with several
//                  it writes its partial tile, summed by stats_finish.
//                * request chunk: LDS histograms of up to kReqChunk requests
//                  (one binary search over the request offsets per token).
//                Token ids are staged through LDS with all of a thread's loads
//                in flight at once, so a block pays about one memory latency
//                per 4096 ids.
//   stats_finish grid (affinity chunks + 1 + 64-expert chunks) x layers:
//                sums the split partials (affinity, counts, union), and the
//                document frequency over the requests, idf = ln(R/df) in
//                double (or the caller's idf) and the signature.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kAffRows = 16;          // affinity rows per tile with a single split
constexpr int kLdsInts = kAffRows * MOE_MAX_EXPERTS_DEV;   // 32 KiB of LDS counters per block
constexpr int kReqChunk = 8;          // requests per histogram block
constexpr int kIdsBuf = 4096;         // staged token ids per stage
constexpr int kMaxSplits = 32;
constexpr long long kMaxPartialBytes = 256LL << 20;
constexpr int kFinishElems = 4 * kThreads;   // affinity elements summed per block

struct StatsGeom {
  int aff_tiles, rows_per_tile, splits, split_tokens, req_chunks, rc, aff_chunks;
};

// Token splits: one per 4096 ids (at most kMaxSplits), fewer when the partial
// tiles would exceed kMaxPartialBytes.  Depends on host-known sizes only, so
// the workspace query can size the partials.
int split_count(int L, int T, int k, int E) {
  long long s = (1LL * T * k + kIdsBuf - 1) / kIdsBuf;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  const long long per = 1LL * L * (1LL * E * E + E) * 4;
  while (s > 1 && s * per > kMaxPartialBytes) --s;
  return static_cast<int>(s);
}

StatsGeom geometry(int L, int T, int k, int E, int R, bool want_aff, bool want_req) {
  StatsGeom g;
  // Every affinity block scans all ids of its split, so with several splits
  // the tiles are as tall as the LDS counters allow (fewer redundant scans);
  // a single split keeps 16-row tiles so a small batch still spreads over
  // several blocks.
  g.splits = split_count(L, T, k, E);
  const int tall = E < kLdsInts / E ? E : kLdsInts / E;
  g.rows_per_tile = !want_aff ? E : g.splits > 1 ? tall : (E < kAffRows ? E : kAffRows);
  g.aff_tiles = want_aff ? (E + g.rows_per_tile - 1) / g.rows_per_tile : 1;
  g.split_tokens = (T + g.splits - 1) / g.splits;
  g.rc = kLdsInts / E;
  if (g.rc > kReqChunk) g.rc = kReqChunk;
  g.req_chunks = want_req && R > 0 ? (R + g.rc - 1) / g.rc : 0;
  g.aff_chunks = g.splits > 1 && want_aff ? (E * E + kFinishElems - 1) / kFinishElems : 0;
  return g;
}

// Stage ids [first, first + n) of one layer into idbuf (clamped to [0, E)).
// Every load of a thread is issued before any is used.
__device__ __forceinline__ void stage_ids(int* idbuf, const int* __restrict__ lid, int first, int n, int E) {
  constexpr int kPer = kIdsBuf / kThreads;
  int v[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = threadIdx.x + q * kThreads;
    v[q] = i < n ? lid[first + i] : 0;
  }
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = threadIdx.x + q * kThreads;
    if (i < n) idbuf[i] = clamp_id(v[q], E);
  }
}

__global__ __launch_bounds__(kThreads) void stats_count(const int* __restrict__ ids, int L, int T, int k, int E,
                                                        StatsGeom geo, int* __restrict__ counts,
                                                        int* __restrict__ union_size,
                                                        uint8_t* __restrict__ union_mask, int* __restrict__ affinity,
                                                        const int* __restrict__ req_offsets, int R,
                                                        int* __restrict__ req_counts, int* __restrict__ part_aff,
                                                        int* __restrict__ part_cnt) {
  __shared__ int lds[kLdsInts];
  __shared__ int cnt[MOE_MAX_EXPERTS_DEV];
  __shared__ int offs[kReqChunk + 1];
  __shared__ int red[kThreads / kWave];
  __shared__ int idbuf[kIdsBuf];
  const int l = blockIdx.y;
  const int* lid = ids + static_cast<size_t>(l) * T * k;
  const int tb = kIdsBuf / k;            // tokens per stage (k <= 512)

  if (static_cast<int>(blockIdx.x) >= geo.aff_tiles * geo.splits) {
    // ---- request chunk: histograms of requests [r0, r0 + nr) ----
    const int r0 = (blockIdx.x - geo.aff_tiles * geo.splits) * geo.rc;
    const int nr = min(geo.rc, R - r0);
    for (int i = threadIdx.x; i < nr * E; i += kThreads) lds[i] = 0;
    for (int i = threadIdx.x; i <= nr; i += kThreads) offs[i] = max(0, min(req_offsets[r0 + i], T));
    __syncthreads();
    const int t_lo = offs[0], t_hi = max(offs[0], offs[nr]);
    for (int ts = t_lo; ts < t_hi; ts += tb) {
      const int nt = min(tb, t_hi - ts);
      __syncthreads();                   // previous stage fully consumed
      stage_ids(idbuf, lid, ts * k, nt * k, E);
      __syncthreads();
      for (int tt = threadIdx.x; tt < nt; tt += kThreads) {
        const int t = ts + tt;
        int lo = 0, hi = nr;             // last r with offs[r] <= t
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (offs[mid] <= t) lo = mid; else hi = mid;
        }
        if (t >= offs[lo + 1]) continue; // not inside request lo (offsets not increasing)
        int* dst = lds + lo * E;
        for (int j = 0; j < k; ++j) atomicAdd(&dst[idbuf[tt * k + j]], 1);
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nr * E; i += kThreads) {
      const int r = r0 + i / E, e = i % E;
      req_counts[(static_cast<size_t>(r) * L + l) * E + e] = lds[i];
    }
    return;
  }

  // ---- affinity tile: rows [a0, a0 + rows) of M^T M over the split's tokens;
  // tile 0 also counts ----
  const int tile = blockIdx.x % geo.aff_tiles, split = blockIdx.x / geo.aff_tiles;
  const int a0 = tile * geo.rows_per_tile;
  const int rows = min(geo.rows_per_tile, E - a0);
  const bool want_aff = affinity != nullptr;
  const bool tile0 = tile == 0;
  const int t_begin = min(T, split * geo.split_tokens), t_end = min(T, t_begin + geo.split_tokens);
  if (want_aff)
    for (int i = threadIdx.x; i < rows * E; i += kThreads) lds[i] = 0;
  for (int e = threadIdx.x; e < E; e += kThreads) cnt[e] = 0;
  for (int t0 = t_begin; t0 < t_end; t0 += tb) {
    const int nt = min(tb, t_end - t0);
    __syncthreads();
    stage_ids(idbuf, lid, t0 * k, nt * k, E);
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
  if (geo.splits > 1) {
    // partial results, summed by stats_finish
    const size_t ps = static_cast<size_t>(split) * L + l;
    if (want_aff) {
      int* dst = part_aff + (ps * E + a0) * E;
      for (int i = threadIdx.x; i < rows * E; i += kThreads) dst[i] = lds[i];
    }
    if (tile0)
      for (int e = threadIdx.x; e < E; e += kThreads) part_cnt[ps * E + e] = cnt[e];
    return;
  }
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

// Block roles, by blockIdx.x:
//   [0, aff_chunks)         kFinishElems affinity entries: sum of the split partials
//   aff_chunks              counts, union mask and union size from the partials
//                           (only when there are several splits)
//   aff_chunks + 1 + c      experts [64c, 64c + 64): df, idf, signature (when wanted)
// In the idf role lanes own an expert and the four waves split the requests;
// loads are issued kBatch at a time so a batch of requests costs one memory
// latency.
constexpr int kBatch = 8;

__global__ __launch_bounds__(kThreads) void stats_finish(int L, int E, int R, StatsGeom geo,
                                                         const int* __restrict__ part_aff,
                                                         const int* __restrict__ part_cnt,
                                                         int* __restrict__ affinity, int* __restrict__ counts,
                                                         int* __restrict__ union_size,
                                                         uint8_t* __restrict__ union_mask,
                                                         const int* __restrict__ req_counts,
                                                         const float* __restrict__ idf_in,
                                                         float* __restrict__ signature) {
  constexpr int kW = kThreads / kWave;
  __shared__ int dfp[kW][kWave];
  __shared__ double idf[kWave];
  __shared__ int red[kW];
  const int l = blockIdx.y;
  const int bx = blockIdx.x;
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const size_t EE = static_cast<size_t>(E) * E;

  if (bx < geo.aff_chunks) {
    const size_t i0 = static_cast<size_t>(bx) * kFinishElems + 4 * threadIdx.x;
    int acc[4] = {0, 0, 0, 0};
    // the split partials are loaded kSplitBatch at a time, all in flight together
    constexpr int kSplitBatch = 8;
    if (i0 + 4 <= EE && EE % 4 == 0 && (reinterpret_cast<uintptr_t>(affinity) & 15) == 0) {
      for (int s0 = 0; s0 < geo.splits; s0 += kSplitBatch) {
        int4 v[kSplitBatch];
#pragma unroll
        for (int b = 0; b < kSplitBatch; ++b)
          v[b] = s0 + b < geo.splits
                     ? *reinterpret_cast<const int4*>(part_aff + (static_cast<size_t>(s0 + b) * L + l) * EE + i0)
                     : make_int4(0, 0, 0, 0);
#pragma unroll
        for (int b = 0; b < kSplitBatch; ++b) {
          acc[0] += v[b].x;
          acc[1] += v[b].y;
          acc[2] += v[b].z;
          acc[3] += v[b].w;
        }
      }
      *reinterpret_cast<int4*>(affinity + l * EE + i0) = make_int4(acc[0], acc[1], acc[2], acc[3]);
    } else {
      for (int q = 0; q < 4; ++q) {
        if (i0 + q >= EE) break;
        int a = 0;
        for (int s = 0; s < geo.splits; ++s) a += part_aff[(static_cast<size_t>(s) * L + l) * EE + i0 + q];
        affinity[l * EE + i0 + q] = a;
      }
    }
    return;
  }
  if (bx == geo.aff_chunks) {
    if (geo.splits == 1) return;
    int nz = 0;
    for (int e = threadIdx.x; e < E; e += kThreads) {
      int c = 0;
      for (int s = 0; s < geo.splits; ++s) c += part_cnt[(static_cast<size_t>(s) * L + l) * E + e];
      counts[static_cast<size_t>(l) * E + e] = c;
      if (union_mask) union_mask[static_cast<size_t>(l) * E + e] = c > 0 ? 1 : 0;
      nz += c > 0 ? 1 : 0;
    }
    nz = wave_sum(nz);
    if (lane == 0) red[w] = nz;
    __syncthreads();
    if (threadIdx.x == 0) {
      int s = 0;
      for (int i = 0; i < kW; ++i) s += red[i];
      union_size[l] = s;
    }
    return;
  }
  if (!signature) return;
  const int e = (bx - geo.aff_chunks - 1) * kWave + lane;
  const bool ok = e < E;
  const int ec = ok ? e : 0;
  const size_t rstride = static_cast<size_t>(L) * E;
  const int* base = req_counts + static_cast<size_t>(l) * E + ec;
  // loads below read clamped, always valid addresses and mask the value
  // afterwards: a load under a branch is followed by a wait, which would turn
  // each batch into kBatch memory round trips
  int df = 0;
  if (!idf_in) {
    for (int r0 = w; r0 < R; r0 += kW * kBatch) {
      int v[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) v[b] = base[static_cast<size_t>(min(r0 + b * kW, R - 1)) * rstride];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) df += (ok && r0 + b * kW < R && v[b] > 0) ? 1 : 0;
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
    for (int b = 0; b < kBatch; ++b) v[b] = base[static_cast<size_t>(min(r0 + b * kW, R - 1)) * rstride];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int r = r0 + b * kW;
      if (r < R) sbase[static_cast<size_t>(r) * rstride] = static_cast<float>(static_cast<double>(v[b]) * f);
    }
  }
}

// ---- small batches: one launch, a few 1024-thread blocks per layer ------------
// When the affinity matrix, the request histograms and the request offsets fit
// in 56 KiB of LDS, each block of a layer builds all of them in LDS (the work
// is a few thousand LDS atomics) and writes its share of the output rows, so
// the writes spread over kSmallSplit CUs.  Decode-sized batches: the two-launch
// path would pay a second launch and a global round trip.
// Ids are staged through LDS a chunk at a time (the first chunk's loads are
// issued together with the request offsets', one memory latency); each thread
// takes one (token, slot) pair, so the chains of dependent LDS atomics stay
// short.  The document frequency counts a request for expert e when its
// histogram cell goes from 0 to 1.
constexpr int kSmallThreads = 1024;
constexpr int kSmallLds = 14336;     // ints shared by affinity, request counts, offsets
constexpr int kSmallIds = 4096;      // staged ids per chunk
constexpr int kSmallSplit = 8;       // blocks per layer (each writes an eighth of the rows)

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
  __shared__ int idbuf[kSmallIds];
  __shared__ int reqof[kSmallIds];
  __shared__ int cnt[MOE_MAX_EXPERTS_DEV];
  __shared__ int dfc[MOE_MAX_EXPERTS_DEV];
  __shared__ double idf[MOE_MAX_EXPERTS_DEV];
  __shared__ int red[kSmallThreads / kWave];
  constexpr int kPer = kSmallIds / kSmallThreads;
  const int l = blockIdx.x / kSmallSplit, part = blockIdx.x % kSmallSplit;
  const int tid = threadIdx.x;
  const bool want_aff = affinity != nullptr;
  const bool want_req = req_offsets != nullptr && R > 0 && (req_counts != nullptr || signature != nullptr);
  const bool need_df = want_req && signature && !idf_in;
  int* aff = lds;
  int* req = lds + (want_aff ? E * E : 0);
  int* offs = req + (want_req ? R * E : 0);
  const int* lid = ids + static_cast<size_t>(l) * T * k;
  const int tpc = kSmallIds / k;                       // tokens per chunk (k <= 512)
  // loads of a chunk's ids: clamped addresses, so none waits for another
  int v[kPer];
  auto load_ids = [&](int t0, int n) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) v[q] = lid[static_cast<size_t>(t0) * k + min(tid + q * kSmallThreads, max(n - 1, 0))];
  };
  if (T > 0) load_ids(0, min(tpc, T) * k);
  const int used = (want_aff ? E * E : 0) + (want_req ? R * E : 0);
  for (int i = tid; i < used; i += kSmallThreads) lds[i] = 0;
  for (int e = tid; e < E; e += kSmallThreads) {
    cnt[e] = 0;
    dfc[e] = 0;
  }
  if (want_req)
    for (int i = tid; i <= R; i += kSmallThreads) offs[i] = max(0, min(req_offsets[i], T));
  for (int t0 = 0; t0 < T; t0 += tpc) {
    const int nt = min(tpc, T - t0), n = nt * k;
    if (t0 > 0) load_ids(t0, n);
    __syncthreads();                                   // previous chunk consumed; zeroing and offsets done
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int i = tid + q * kSmallThreads;
      if (i < n) idbuf[i] = clamp_id(v[q], E);
    }
    // request of each token of the chunk (-1: none)
    for (int tt = tid; tt < nt; tt += kSmallThreads) {
      const int t = t0 + tt;
      int r = -1;
      if (want_req && t >= offs[0] && t < offs[R]) {
        int lo = 0, hi = R;                   // last r with offs[r] <= t
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (offs[mid] <= t) lo = mid; else hi = mid;
        }
        if (t < offs[lo + 1]) r = lo;
      }
      reqof[tt] = r;
    }
    __syncthreads();
    for (int i = tid; i < n; i += kSmallThreads) {
      const int tt = i / k;
      const int a = idbuf[i];
      atomicAdd(&cnt[a], 1);
      const int r = reqof[tt];
      if (r >= 0) {
        const int old = atomicAdd(&req[r * E + a], 1);
        if (need_df && old == 0) atomicAdd(&dfc[a], 1);
      }
      if (want_aff) {
        const int* row = idbuf + tt * k;
        int* dst = aff + a * E;
        for (int j2 = 0; j2 < k; ++j2) atomicAdd(&dst[row[j2]], 1);
      }
    }
  }
  __syncthreads();
  // rows [lo, hi) of E (affinity) and of R (requests) are this block's to write
  auto share = [&](int n, int& lo, int& hi) {
    const int per = (n + kSmallSplit - 1) / kSmallSplit;
    lo = min(n, part * per);
    hi = min(n, lo + per);
  };
  if (part == 0) {
    int nz = 0;
    for (int e = tid; e < E; e += kSmallThreads) {
      const int c = cnt[e];
      counts[static_cast<size_t>(l) * E + e] = c;
      if (union_mask) union_mask[static_cast<size_t>(l) * E + e] = c > 0 ? 1 : 0;
      nz += c > 0 ? 1 : 0;
    }
    nz = wave_sum(nz);
    if (lane_id() == 0) red[tid >> 6] = nz;
  }
  if (want_aff) {
    int a_lo, a_hi;
    share(E, a_lo, a_hi);
    int* dst = affinity + static_cast<size_t>(l) * E * E;
    for (int i = a_lo * E + tid; i < a_hi * E; i += kSmallThreads) dst[i] = aff[i];
  }
  if (signature && want_req)
    for (int e = tid; e < E; e += kSmallThreads) {
      if (idf_in) {
        idf[e] = static_cast<double>(idf_in[static_cast<size_t>(l) * E + e]);
      } else {
        const int df = dfc[e];
        idf[e] = df > 0 ? log(static_cast<double>(R) / static_cast<double>(df)) : 0.0;
      }
    }
  __syncthreads();
  if (part == 0 && tid == 0) {
    int sum = 0;
    for (int w = 0; w < kSmallThreads / kWave; ++w) sum += red[w];
    union_size[l] = sum;
  }
  if (!want_req) return;
  int r_lo, r_hi;
  share(R, r_lo, r_hi);
  for (int i = r_lo * E + tid; i < r_hi * E; i += kSmallThreads) {
    const int rr = i / E, e = i % E;
    const size_t at = (static_cast<size_t>(rr) * L + l) * E + e;
    if (req_counts) req_counts[at] = req[i];
    if (signature) signature[at] = static_cast<float>(static_cast<double>(req[i]) * idf[e]);
  }
}

struct WsLayout {
  size_t rc_off, aff_off, cnt_off, total;
};

WsLayout ws_layout(int L, int T, int k, int E, int R) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  const int S = split_count(L, T, k, E);
  WsLayout w;
  w.rc_off = 0;
  w.aff_off = up(static_cast<size_t>(R) * L * E * 4);
  const size_t aff = S > 1 ? static_cast<size_t>(S) * L * E * E * 4 : 0;
  w.cnt_off = w.aff_off + up(aff);
  const size_t cnt = S > 1 ? static_cast<size_t>(S) * L * E * 4 : 0;
  w.total = w.cnt_off + up(cnt) + 256;
  return w;
}

}  // namespace

size_t stats_workspace_bytes(int L, int T, int k, int E, int R) { return ws_layout(L, T, k, E, R).total; }

hipError_t launch_stats(const StatsArgs& a, void* workspace, hipStream_t stream) {
  if (a.L == 0) return hipSuccess;
  const bool want_req = a.req_offsets && a.R > 0 && (a.req_counts || a.signature);
  if (small_fits(a.E, a.R, a.affinity != nullptr, want_req, a.T, a.k)) {
    hipLaunchKernelGGL(stats_small, dim3(a.L * kSmallSplit), dim3(kSmallThreads), 0, stream, a.topk_ids, a.L, a.T, a.k, a.E,
                       a.counts, a.union_size, a.union_mask, a.affinity, want_req ? a.req_offsets : nullptr,
                       want_req ? a.R : 0, a.idf, a.req_counts, a.signature);
    return hipGetLastError();
  }
  const StatsGeom geo = geometry(a.L, a.T, a.k, a.E, a.R, a.affinity != nullptr, want_req);
  const WsLayout w = ws_layout(a.L, a.T, a.k, a.E, a.R);
  char* ws = static_cast<char*>(workspace);
  int* rc = a.req_counts ? a.req_counts : reinterpret_cast<int*>(ws + w.rc_off);
  int* part_aff = reinterpret_cast<int*>(ws + w.aff_off);
  int* part_cnt = reinterpret_cast<int*>(ws + w.cnt_off);
  hipLaunchKernelGGL(stats_count, dim3(geo.aff_tiles * geo.splits + geo.req_chunks, a.L), dim3(kThreads), 0, stream,
                     a.topk_ids, a.L, a.T, a.k, a.E, geo, a.counts, a.union_size, a.union_mask, a.affinity,
                     a.req_offsets, a.R, rc, part_aff, part_cnt);
  const bool sig = want_req && a.signature;
  if (geo.splits > 1 || sig) {
    const int blocks = geo.aff_chunks + 1 + (sig ? (a.E + kWave - 1) / kWave : 0);
    hipLaunchKernelGGL(stats_finish, dim3(blocks, a.L), dim3(kThreads), 0, stream, a.L, a.E, a.R, geo,
                       static_cast<const int*>(part_aff), static_cast<const int*>(part_cnt), a.affinity, a.counts,
                       a.union_size, a.union_mask, static_cast<const int*>(rc), a.idf, sig ? a.signature : nullptr);
  }
  return hipGetLastError();
}

}  // namespace moe
