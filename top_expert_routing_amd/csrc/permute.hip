// Dispatch permutation: stable counting sort of the token->expert assignments
// into contiguous groups, then a gather of the token rows.
//
// GRACE-MoE page, section 1: the dispatch exchange sends each token to its
// experts; on one GPU it becomes this regrouping.  Ordering is (group, flat
// index), so the result is unique and the kernels must be stable.
//
// Assignments are cut into chunks of kChunk; each 256-thread block owns one
// chunk and each of its four waves a contiguous quarter.  A wave ranks 64
// consecutive assignments at a time: a bitwise ballot "match" gives every lane
// the set of lanes with the same group, the rank inside the wave is the
// popcount of the lower matching lanes, and the lowest matching lane carries
// the running per-group counter.  Block bases come from an exclusive scan over
// (group, chunk) in group-major order, so positions are stable across chunks.
// Small batches (<= 4096 routed assignments) take a one-launch path in which
// every block recomputes the histogram it needs (see permute_small).
// Shared-expert assignments are already in sorted order (f = T*k + s*T + t is
// the position itself), so they are written directly.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kPerWave = 256;
constexpr int kChunk = kWaves * kPerWave;   // 1024 assignments per block
constexpr int kMaxRoutedGroups = 2 * 512;   // nseg * E

struct PermCtx {
  const int* ids;
  int T, E, k, n_priority, Nr, Gr, nbits, nb;
};

__device__ __forceinline__ int group_of(const PermCtx& c, int i) {
  const int t = i / c.k;
  const int e = clamp_id(c.ids[i], c.E);
  const int seg = (c.n_priority > 0 && t >= c.n_priority) ? 1 : 0;
  return seg * c.E + e;
}

// Lanes of this wave holding the same key (all 64 lanes must call).
__device__ __forceinline__ uint64_t match_any(int key, int nbits) {
  uint64_t m = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    const int bit = (key >> b) & 1;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Each lane keeps the groups of its (up to) kIters assignments of the chunk in
// registers: loaded once, used by the histogram and by the scatter pass.
constexpr int kIters = kPerWave / kWave;   // 4

__device__ __forceinline__ void load_groups(const PermCtx& c, int b, int (&grp)[kIters]) {
  const int w = threadIdx.x >> 6, lane = lane_id();
  const int i0 = b * kChunk + w * kPerWave;
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int i = i0 + it * kWave + lane;
    grp[it] = i < c.Nr ? group_of(c, i) : c.Gr;    // c.Gr: sentinel, matches no real group
  }
}

// Histogram of one chunk into wave-private counters (pass 1).
__device__ __forceinline__ void chunk_histogram(const PermCtx& c, int b, const int (&grp)[kIters], int* wcnt) {
  const int w = threadIdx.x >> 6, lane = lane_id();
  for (int g = lane; g < c.Gr; g += kWave) wcnt[w * kMaxRoutedGroups + g] = 0;
  const int i0 = b * kChunk + w * kPerWave;
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    if (i0 + it * kWave >= c.Nr) break;               // wave-uniform
    const int g = grp[it];
    const uint64_t m = match_any(g, c.nbits);
    if (g < c.Gr && (__ffsll(static_cast<unsigned long long>(m)) - 1) == lane)
      wcnt[w * kMaxRoutedGroups + g] += __popcll(static_cast<unsigned long long>(m));
  }
}

// Ranks and scatter (pass 3): wcnt holds each wave's running base per group.
// Only the leader lane of a group touches its counter; a wave's LDS accesses
// execute in program order, so the next leader of that group reads the
// updated value.  The counters are plain LDS (not volatile): a volatile access
// through a generic pointer becomes a flat access that waits on every
// outstanding global store.
__device__ __forceinline__ void chunk_scatter(const PermCtx& c, int b, const int (&grp)[kIters], int* wcnt, int* s2f,
                                              int* f2s, int* tok) {
  const int w = threadIdx.x >> 6, lane = lane_id();
  const int i0 = b * kChunk + w * kPerWave;
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    if (i0 + it * kWave >= c.Nr) break;
    const int i = i0 + it * kWave + lane;
    const int g = grp[it];
    const bool valid = g < c.Gr;
    const uint64_t m = match_any(g, c.nbits);
    const int leader = __ffsll(static_cast<unsigned long long>(m)) - 1;
    int base = 0;
    if (valid && leader == lane) {
      base = wcnt[w * kMaxRoutedGroups + g];
      wcnt[w * kMaxRoutedGroups + g] = base + __popcll(static_cast<unsigned long long>(m));
    }
    base = __shfl(base, leader, kWave);
    if (valid) {
      const int pos = base + __popcll(static_cast<unsigned long long>(m & lanemask_lt()));
      s2f[pos] = i;
      f2s[i] = pos;
      if (tok) tok[pos] = i / c.k;
    }
  }
}

// Shared-expert assignments sit at their own flat index.
__device__ __forceinline__ void write_shared_identity(int Nr, int N, int T, int nblocks, int b, int* s2f, int* f2s,
                                                      int* tok) {
  for (int f = Nr + b * kThreads + threadIdx.x; f < N; f += nblocks * kThreads) {
    s2f[f] = f;
    f2s[f] = f;
    if (tok) tok[f] = (f - Nr) % T;
  }
}

// Exclusive scan of per-thread values across the block; returns the prefix
// and stores the total in *total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) scratch[w] = incl;
  __syncthreads();
  int wbase = 0, tot = 0;
  for (int i = 0; i < kWaves; ++i) {
    if (i < w) wbase += scratch[i];
    tot += scratch[i];
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
}

// Copy rows src_row(j) -> dst_row(j) for j < nrows, kCopyRows rows at a time:
// a thread owns one 16-byte column of the rows, so its kCopyRows loads are in
// flight together and consecutive threads touch consecutive bytes of a row.
constexpr int kCopyRows = 16;

template <typename SrcRow, typename DstRow>
__device__ __forceinline__ void copy_rows(const uint4* __restrict__ x, uint4* __restrict__ xs, int nrows,
                                          int row_vecs, SrcRow src_row, DstRow dst_row) {
  for (int j0 = 0; j0 < nrows; j0 += kCopyRows) {
    const int nr = min(kCopyRows, nrows - j0);
    const uint4* src[kCopyRows];
    uint4* dst[kCopyRows];
#pragma unroll
    for (int j = 0; j < kCopyRows; ++j) {
      const int jj = j0 + (j < nr ? j : 0);
      src[j] = x + static_cast<size_t>(src_row(jj)) * row_vecs;
      dst[j] = xs + static_cast<size_t>(dst_row(jj)) * row_vecs;
    }
    for (int c = threadIdx.x; c < row_vecs; c += kThreads) {
      // every load is issued (rows past nr re-read row j0): a load under a
      // branch is followed by a wait, which would serialise the 16 loads
      uint4 v[kCopyRows];
#pragma unroll
      for (int j = 0; j < kCopyRows; ++j) v[j] = src[j][c];
#pragma unroll
      for (int j = 0; j < kCopyRows; ++j)
        if (j < nr) dst[j][c] = v[j];
    }
  }
}

// ---- small batches: one launch, many blocks, no inter-block communication ----
// Block b ranks assignments [16b, 16b+16).  Every block builds the histogram of
// all routed assignments and of those before its chunk (the whole id array is
// a few KiB and sits in L2), so it knows its group bases without waiting for
// any other block.  One wave ranks the chunk with a ballot match; then the four
// waves gather the chunk's token rows.  Shared-expert rows are split evenly
// over the blocks.
constexpr int kSmallChunk = 16;   // assignments ranked (and rows gathered) per block
constexpr int kSmallMaxNr = 4096;

__global__ __launch_bounds__(kThreads) void permute_small(PermCtx c, int n_shared, int* __restrict__ group_offsets,
                                                          int* __restrict__ s2f, int* __restrict__ f2s,
                                                          int* __restrict__ tok,
                                                          const uint4* __restrict__ x, int row_vecs,
                                                          uint4* __restrict__ xs) {
  __shared__ int total[kMaxRoutedGroups];
  __shared__ int before[kMaxRoutedGroups];
  __shared__ int scratch[kWaves];
  __shared__ int pos_s[kSmallChunk];
  __shared__ int tok_s[kSmallChunk];
  const int b = blockIdx.x, nb = gridDim.x;
  const int lo = b * kSmallChunk, hi = min(c.Nr, lo + kSmallChunk);
  for (int g = threadIdx.x; g < c.Gr; g += kThreads) {
    total[g] = 0;
    before[g] = 0;
  }
  __syncthreads();
  {
    // all of a thread's id loads are issued before its first atomic
    constexpr int kPer = kSmallMaxNr / kThreads;
    int gq[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int i = threadIdx.x + q * kThreads;
      gq[q] = i < c.Nr ? group_of(c, i) : -1;
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int i = threadIdx.x + q * kThreads;
      if (gq[q] < 0) continue;
      atomicAdd(&total[gq[q]], 1);
      if (i < lo) atomicAdd(&before[gq[q]], 1);
    }
  }
  __syncthreads();
  // exclusive scan of the totals: thread owns 4 consecutive groups
  constexpr int kPer = kMaxRoutedGroups / kThreads;
  int own[kPer];
  int sum = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int g = threadIdx.x * kPer + q;
    own[q] = g < c.Gr ? total[g] : 0;
    sum += own[q];
  }
  int tot;
  int run = block_exclusive_scan(sum, scratch, &tot);
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int g = threadIdx.x * kPer + q;
    if (g < c.Gr) {
      before[g] += run;                 // now: first sorted row of this chunk's part of group g
      if (b == 0) group_offsets[g] = run;
    }
    run += own[q];
  }
  if (b == 0)
    for (int s = threadIdx.x; s <= n_shared; s += kThreads) group_offsets[c.Gr + s] = c.Nr + s * c.T;
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int i = lo + lane;
    const bool valid = i < hi;
    const int g = valid ? group_of(c, i) : c.Gr;
    const uint64_t m = match_any(g, c.nbits);
    int pos = -1;
    if (valid) {
      pos = before[g] + __popcll(static_cast<unsigned long long>(m & lanemask_lt()));
      s2f[pos] = i;
      f2s[i] = pos;
      if (tok) tok[pos] = i / c.k;
    }
    pos_s[lane] = pos;
    tok_s[lane] = valid ? i / c.k : 0;
  }
  // shared-expert rows [Nr + b*per, ...): position == flat index
  const int N = c.Nr + n_shared * c.T;
  const int sper = (N - c.Nr + nb - 1) / nb;
  const int s_lo = c.Nr + b * sper, s_hi = min(N, s_lo + sper);
  for (int f = s_lo + threadIdx.x; f < s_hi; f += kThreads) {
    s2f[f] = f;
    f2s[f] = f;
    if (tok) tok[f] = (f - c.Nr) % c.T;
  }
  __syncthreads();
  if (x == nullptr) return;
  const int nvalid = hi > lo ? hi - lo : 0;        // chunk entries are a prefix of pos_s
  copy_rows(x, xs, nvalid, row_vecs, [&](int j) { return tok_s[j]; }, [&](int j) { return pos_s[j]; });
  copy_rows(x, xs, s_hi > s_lo ? s_hi - s_lo : 0, row_vecs, [&](int j) { return (s_lo + j - c.Nr) % c.T; },
            [&](int j) { return s_lo + j; });
}

// ---- several chunks: count, scan, scatter -----------------------------------
__global__ __launch_bounds__(kThreads) void permute_count(PermCtx c, int* blk) {
  __shared__ int hist[kMaxRoutedGroups];
  for (int g = threadIdx.x; g < c.Gr; g += kThreads) hist[g] = 0;
  __syncthreads();
  const int b = blockIdx.x;
  const int lo = b * kChunk, hi = min(c.Nr, lo + kChunk);
  for (int i = lo + threadIdx.x; i < hi; i += kThreads) atomicAdd(&hist[group_of(c, i)], 1);
  __syncthreads();
  for (int g = threadIdx.x; g < c.Gr; g += kThreads) blk[g * c.nb + b] = hist[g];
}

__global__ __launch_bounds__(1024) void permute_scan(PermCtx c, int n_shared, int* blk, int* group_offsets) {
  __shared__ int part[1024];
  // a thread's counts are read kBatch at a time from clamped addresses, all in
  // flight together (loads under a bounds test would each wait for the last)
  constexpr int kBatch = 8;
  const int M = c.Gr * c.nb;
  const int per = (M + 1023) / 1024;
  const int lo = threadIdx.x * per, hi = min(M, lo + per);
  int s = 0;
  for (int i0 = lo; i0 < hi; i0 += kBatch) {
    int v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) v[b] = blk[min(i0 + b, M - 1)];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) s += i0 + b < hi ? v[b] : 0;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 partial sums
  for (int o = 1; o < 1024; o <<= 1) {
    int v = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = part[threadIdx.x] - s;
  for (int i0 = lo; i0 < hi; i0 += kBatch) {
    int v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) v[b] = blk[min(i0 + b, M - 1)];   // entries past hi are not used
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int i = i0 + b;
      if (i >= hi) break;
      blk[i] = run;
      if (i % c.nb == 0) group_offsets[i / c.nb] = run;
      run += v[b];
    }
  }
  for (int q = threadIdx.x; q <= n_shared; q += 1024) group_offsets[c.Gr + q] = c.Nr + q * c.T;
}

// SCAN = false: blk holds the scanned bases (permute_scan ran).  SCAN = true
// (at most kMaxNbFused chunks): blk holds the raw per-chunk counts and every
// block derives its bases itself - a group's base is the sum of all counts of
// the groups before it, plus the group's counts in the chunks before this one
// - so no scan launch is needed; block 0 writes group_offsets.
constexpr int kMaxNbFused = 64;
constexpr int kGroupsPerThread = kMaxRoutedGroups / kThreads;   // 4

template <bool SCAN>
__global__ __launch_bounds__(kThreads) void permute_scatter(PermCtx c, int n_shared, const int* blk, int* s2f,
                                                            int* f2s, int* tok, int* group_offsets) {
  __shared__ int wcnt[kWaves * kMaxRoutedGroups];
  __shared__ int wsum[kWaves];
  int* vw = wcnt;
  const int b = blockIdx.x;
  int grp[kIters];
  load_groups(c, b, grp);
  chunk_histogram(c, b, grp, vw);
  // base[q]: this block's first sorted position of group tid * GPT + q
  int base[kGroupsPerThread];
  const int GPT = (c.Gr + kThreads - 1) / kThreads;
  const int g0 = threadIdx.x * GPT;
  if constexpr (SCAN) {
    int tot[kGroupsPerThread], pre[kGroupsPerThread];
    int sum = 0;
#pragma unroll
    for (int q = 0; q < kGroupsPerThread; ++q) {
      tot[q] = pre[q] = 0;
      const int g = g0 + q;
      if (q < GPT && g < c.Gr) {
        // all of the group's chunk counts in flight at once (clamped addresses)
        int v[kMaxNbFused];
#pragma unroll
        for (int i = 0; i < kMaxNbFused; ++i) v[i] = blk[g * c.nb + min(i, c.nb - 1)];
#pragma unroll
        for (int i = 0; i < kMaxNbFused; ++i) {
          const int x = i < c.nb ? v[i] : 0;
          tot[q] += x;
          pre[q] += i < b ? x : 0;
        }
      }
      sum += tot[q];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o, kWave);
      if (lane_id() >= o) incl += y;
    }
    if (lane_id() == kWave - 1) wsum[threadIdx.x >> 6] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < (static_cast<int>(threadIdx.x) >> 6); ++w) run += wsum[w];
#pragma unroll
    for (int q = 0; q < kGroupsPerThread; ++q) {
      const int g = g0 + q;
      if (b == 0 && q < GPT && g < c.Gr) group_offsets[g] = run;
      base[q] = run + pre[q];
      run += tot[q];
    }
    if (b == 0)
      for (int q = threadIdx.x; q <= n_shared; q += kThreads) group_offsets[c.Gr + q] = c.Nr + q * c.T;
  } else {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kGroupsPerThread; ++q) {
      const int g = g0 + q;
      base[q] = q < GPT && g < c.Gr ? blk[g * c.nb + b] : 0;
    }
  }
#pragma unroll
  for (int q = 0; q < kGroupsPerThread; ++q) {
    const int g = g0 + q;
    if (q >= GPT || g >= c.Gr) continue;
    int r = base[q];
    for (int w = 0; w < kWaves; ++w) {
      const int cnt = vw[w * kMaxRoutedGroups + g];
      vw[w * kMaxRoutedGroups + g] = r;
      r += cnt;
    }
  }
  __syncthreads();
  chunk_scatter(c, b, grp, vw, s2f, f2s, tok);
  write_shared_identity(c.Nr, c.Nr + n_shared * c.T, c.T, c.nb, b, s2f, f2s, tok);
}

// ---- row gather: x_sorted[n] = x[token(sorted_to_flat[n])] ---------------------
// Each block copies kGatherRows consecutive sorted rows.
constexpr int kGatherRows = kCopyRows;

__global__ __launch_bounds__(kThreads) void permute_gather(const uint4* __restrict__ x, const int* __restrict__ s2f,
                                                           int T, int k, int Nr, int N, int row_vecs,
                                                           uint4* __restrict__ xs) {
  __shared__ int tok[kGatherRows];
  const int n0 = blockIdx.x * kGatherRows;
  const int nr = min(kGatherRows, N - n0);
  if (threadIdx.x < nr) {
    const int f = s2f[n0 + threadIdx.x];
    tok[threadIdx.x] = f < Nr ? f / k : (f - Nr) % T;
  }
  __syncthreads();
  copy_rows(x, xs, nr, row_vecs, [&](int j) { return tok[j]; }, [&](int j) { return n0 + j; });
}

int bits_for(int v) {
  int b = 0;
  while ((1 << b) <= v) ++b;
  return b;
}

PermCtx make_ctx(const PermuteArgs& a) {
  PermCtx c;
  c.ids = a.topk_ids;
  c.T = a.T;
  c.E = a.E;
  c.k = a.k;
  c.n_priority = a.n_priority;
  c.Nr = a.T * a.k;
  c.Gr = (a.n_priority > 0 ? 2 : 1) * a.E;
  c.nbits = bits_for(c.Gr);
  c.nb = c.Nr > 0 ? (c.Nr + kChunk - 1) / kChunk : 1;
  return c;
}

}  // namespace

size_t permute_workspace_bytes(int T, int E, int k, int n_shared, int n_priority) {
  (void)n_shared;
  const long long Nr = static_cast<long long>(T) * k;
  const long long nb = Nr > 0 ? (Nr + kChunk - 1) / kChunk : 1;
  const long long Gr = static_cast<long long>(n_priority > 0 ? 2 : 1) * E;
  if (Nr <= kSmallMaxNr) return 256;   // the one-launch path uses no workspace
  return static_cast<size_t>(((Gr * nb * 4) + 255) / 256 * 256);
}

hipError_t launch_permute(const PermuteArgs& a, void* workspace, hipStream_t stream) {
  const PermCtx c = make_ctx(a);
  const int N = c.Nr + a.n_shared * a.T;
  const int row_vecs = a.x != nullptr ? a.d * a.elem_bytes / 16 : 0;
  if (c.Nr <= kSmallMaxNr) {
    // one launch: ranks, scatter and row gather together
    const int nb = c.Nr > 0 ? (c.Nr + kSmallChunk - 1) / kSmallChunk : 1;
    hipLaunchKernelGGL(permute_small, dim3(nb), dim3(kThreads), 0, stream, c, a.n_shared, a.group_offsets,
                       a.sorted_to_flat, a.flat_to_sorted, a.sorted_token, static_cast<const uint4*>(a.x), row_vecs,
                       static_cast<uint4*>(a.x_sorted));
    return hipGetLastError();
  }
  int* blk = static_cast<int*>(workspace);
  hipLaunchKernelGGL(permute_count, dim3(c.nb), dim3(kThreads), 0, stream, c, blk);
  if (c.nb <= kMaxNbFused) {
    hipLaunchKernelGGL(permute_scatter<true>, dim3(c.nb), dim3(kThreads), 0, stream, c, a.n_shared,
                       static_cast<const int*>(blk), a.sorted_to_flat, a.flat_to_sorted, a.sorted_token,
                       a.group_offsets);
  } else {
    hipLaunchKernelGGL(permute_scan, dim3(1), dim3(1024), 0, stream, c, a.n_shared, blk, a.group_offsets);
    hipLaunchKernelGGL(permute_scatter<false>, dim3(c.nb), dim3(kThreads), 0, stream, c, a.n_shared,
                       static_cast<const int*>(blk), a.sorted_to_flat, a.flat_to_sorted, a.sorted_token,
                       a.group_offsets);
  }
  if (a.x != nullptr && N > 0) {
    const int blocks = (N + kGatherRows - 1) / kGatherRows;
    hipLaunchKernelGGL(permute_gather, dim3(blocks), dim3(kThreads), 0, stream, static_cast<const uint4*>(a.x),
                       a.sorted_to_flat, a.T, a.k, c.Nr, N, row_vecs, static_cast<uint4*>(a.x_sorted));
  }
  return hipGetLastError();
}

}  // namespace moe
