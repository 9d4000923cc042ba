// Grouped SwiGLU expert FFN on bf16 MFMA (gfx950), plus an fp32 path.
//
// ExpertPlex page, "Instance vs module disaggregation": the expert FFN is the
// bulk of a MoE layer; ELDR page, "What it solves": a decode step must read the
// weights of every distinct expert the batch selected - and only those.
//
// Work is cut into tiles (group, block of rows, block of output columns).  The
// tiles are enumerated on the device from group_offsets (empty groups give no
// tiles, so unused experts' weights are never read) and run the two phases:
//   phase 1  a[n][i] = silu(xs[n] . W_gate[e][i]) * (xs[n] . W_up[e][i])  -> bf16
//   phase 2  h[n][o] = a[n] . W_down[e][o]
// either as two launches, or (mixed batches with a priority segment) in one
// persistent launch whose phase-2 tiles wait for their rows' phase-1 tiles.
// Both phases are C = A B^T with A and B contiguous along K, the operand
// layout of the bf16 MFMAs: each lane holds 8 consecutive K values of one row
// of A and of one row of B.  Decode-sized tiles stage the few token rows (A)
// in LDS and stream the weight rows (B), each used by one wave, straight from
// HBM into registers; prefill-sized tiles bring both operands into an LDS
// ring with LDS-DMA loads.
#include <stdlib.h>

#include <type_traits>

#include "common.h"
#include "item_plan.h"
#include "launch.h"
#include "queue_plan.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
// ---- work items: (m-tile of a group, column chunk) ---------------------------
// Every block finds its own work item from group_offsets: the group sizes
// (<= 1280 groups, 5 per thread) are scanned block-wide into m-tile counts, so
// no planning launch and no tile list in memory are needed.  group_offsets is
// a precondition (non-decreasing, last entry n_rows); rows are still clamped to
// [0, n_rows] so a bad input cannot make a tile reach outside the buffers.
//
// Workgroups are dealt round-robin to the 8 XCDs (blockIdx % 8).  The
// (group g, column chunk j) pairs are dealt to the XCDs in turn: pair
// p = g * nch + j goes to XCD p % 8, with all of its m-tiles.  XCD x runs its
// pairs in group order, chunk order, m-tile order, so the m-tiles that share
// a weight slab run together in one L2, every XCD gets a similar mix of large
// and small groups (a hot expert's chunks spread over all eight), and the
// priority segment's items start first on every XCD.
constexpr int kMaxGroups = 2 * 512 + 256;   // nseg * E + shared experts, at most
constexpr int kMaxGroupsPerThread = (kMaxGroups + kThreads - 1) / kThreads;   // for 256 threads

struct PlanArgs {
  const int* offs;
  int G, E, nseg, BM, n_rows, max_tiles;
  int* diag;          // diagnostic word, cleared by block 0 (nullptr: leave it)
  const int* arows;   // A row of sorted row n (nullptr: row n itself)
  int n_x;            // rows of A when arows is given
  float* zero = nullptr;   // zero_n4 float4s the launch's blocks clear (the fused combine's sums)
  int zero_n4 = 0;
};

// The combine folded into the down projection's epilogue (GRACE-MoE page,
// section 1: the gather back to the tokens after the experts): sorted row n's
// output row, rounded to bf16 like h_sorted, is scaled by its gate weight and
// added into y32[token] with fp32 atomics.  Routed rows: flat index
// f = s2f[n] < T*k, token f / k, weight topk_w[f]; shared rows: token
// (f - T*k) mod T, weight 1.
struct CombineArgs {
  const int* s2f;
  const float* topk_w;
  int T, k, n;        // n = T * (k + shared experts) sorted rows
  float* y32;         // [T][d] fp32, zero before the down projection
};

__device__ __forceinline__ void clear_span(const PlanArgs& plan) {
  if (!plan.zero) return;
  float4* z = reinterpret_cast<float4*>(plan.zero);
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < plan.zero_n4; i += gridDim.x * blockDim.x)
    z[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__device__ __forceinline__ float bf16_rne(float v) {
  return __uint_as_float((pack_bf16x2(v, 0.f) & 0xffffu) << 16);
}

// Adds the four columns n..n+3 of sorted row `row` (bf16-rounded, times its
// gate weight) into its token's row of the combine sums.
__device__ __forceinline__ void combine_add4(const CombineArgs& c, int row, int Ncols, int n, const float (&v)[4]) {
  const int f = min(max(c.s2f[row], 0), c.n - 1);     // a bad entry stays inside y32
  const int tk = c.T * c.k;
  const int tok = f < tk ? f / c.k : (f - tk) % c.T;
  const float w = f < tk ? c.topk_w[f] : 1.0f;
  float* y = c.y32 + static_cast<size_t>(tok) * Ncols + n;
#pragma unroll
  for (int t = 0; t < 4; ++t) atomicAdd(y + t, w * bf16_rne(v[t]));
}

// Row of the A matrix that sorted row n reads (the row gather folded into the
// loads when a row list is given; clamped so a bad entry stays in bounds).
__device__ __forceinline__ size_t a_row(const int* arows, int n_x, int n) {
  return arows ? static_cast<size_t>(min(max(arows[n], 0), n_x - 1)) : static_cast<size_t>(n);
}

// a_row of N sorted rows at once: the (wave-uniform) test of the row list is
// taken once, so the N loads are issued back to back and cost one memory
// round trip (with the test inside each a_row call the compiler waits for
// every load before the next).
template <int N>
__device__ __forceinline__ void a_rows(const int* arows, int n_x, const int (&n)[N], size_t (&out)[N]) {
  if (arows) {
    int v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = arows[n[i]];
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = static_cast<size_t>(min(max(v[i], 0), n_x - 1));
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = static_cast<size_t>(n[i]);
  }
}

// Row-list entries of N sorted rows, loaded without a branch (from `dummy`, any
// readable int, when there is no list) so that nothing waits for them before
// a_row_of uses the values.
template <int N>
__device__ __forceinline__ void a_rows_raw(const int* arows, const int* dummy, const int (&n)[N], int (&raw)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) raw[i] = *(arows ? arows + n[i] : dummy);
}
__device__ __forceinline__ size_t a_row_of(const int* arows, int n_x, int n, int raw) {
  return arows ? static_cast<size_t>(min(max(raw, 0), n_x - 1)) : static_cast<size_t>(n);
}

// Must be called by all NT threads of the block.
template <int NT = kThreads>
__device__ Item block_find_item(const PlanArgs& p, int nch) {
  constexpr int GPT = (kMaxGroups + NT - 1) / NT;   // groups per thread
  __shared__ int wsum[NT / kWave];
  __shared__ Item found;
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  const int x = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;               // this block's item within XCD x's list
  if (tid == 0) found = Item{0, 0, 0, 0, 0, 0};
  if (tid == 0 && blockIdx.x == 0 && p.diag) *p.diag = 0;
  GroupRows gr[GPT];
  int s = 0;
#pragma unroll
  for (int q = 0; q < GPT; ++q) {
    const int g = tid * GPT + q;
    gr[q] = GroupRows{0, 0, 0, 0, 0, 0};
    if (g < p.G) {
      gr[q] = group_rows(p.offs, p.n_rows, p.E, p.nseg, p.BM, g);
      s += group_items(gr[q], g, nch, x);
    }
  }
  int incl = s;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) wsum[w] = incl;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) base += i < w ? wsum[i] : 0;
  int t = base + incl - s;     // XCD x's items before this thread's first group
  if (slot >= t && slot < t + s) {
#pragma unroll
    for (int q = 0; q < GPT; ++q) {
      const int g = tid * GPT + q;
      if (g >= p.G) break;
      const GroupRows& r = gr[q];
      const int n = group_items(r, g, nch, x);
      if (slot >= t && slot < t + n) found = group_item(r, g, nch, x, slot - t, p.BM, p.E, p.nseg);
      t += n;
    }
  }
  __syncthreads();
  return found;
}

// silu(g) * u for the bf16 kernels (their result is rounded to bf16, so the
// hardware reciprocal's 1-ulp error is far below the output precision)
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Four bf16 outputs (8 bytes).  COHERENT: as an agent-scope atomic store
// (written through to the device's coherence point, so a consumer on another
// XCD sees it after its acquire without the producer writing back its L2).
template <bool COHERENT>
__device__ __forceinline__ void store4(uint16_t* p, float a, float b, float c, float d) {
  const uint2 v = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
  if constexpr (COHERENT)
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), __builtin_bit_cast(unsigned long long, v),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *reinterpret_cast<uint2*>(p) = v;
}

// ---- decode-sized tiles: weights stream from HBM straight into MFMA registers ----
// One block of four waves per item (m-tile of <= 16*MF rows, 64*NFC output
// columns).  Each wave computes every row of the m-tile against its own 16*NFC
// columns (phase 1: of W_gate and of W_up).
//   * Weight rows (B) are read exactly once per m-tile, straight into the MFMA
//     B operand: a lane loads 16 bytes of one row; the kDecodeKC/32 K-steps of
//     a chunk are issued back to back, so each row streams in runs of
//     kDecodeKC*2 bytes with many loads in flight.  No LDS round trip.
//   * The few token rows (A) are shared by the four waves: staged through LDS
//     one K-chunk at a time, double buffered, loaded from global while the
//     previous chunk is multiplied.  One barrier per chunk.
// Latency is hidden by the chunk-deep weight loads and the other resident
// blocks (four per CU for tiles of <= 32 rows).
// K per chunk: 256 (8 MFMA K-steps) for tiles of <= 32 rows; the 64-row tile
// (MF = 4) runs at two waves per SIMD and does better with 128 (measured:
// DSv2-Lite-shaped t256 FFN 247.7 -> 244.4 us; OLMoE-shaped 159.7 -> 166.9
// with 128 at MF = 2).
template <int MF>
constexpr int decode_kc() { return MF <= 2 ? 256 : 128; }
constexpr int kDecodeWavesPerSimd = 4;

// LDS staging of one decode tile: two buffers of BM rows x (KC + 8) bf16.
template <int MF>
constexpr int decode_lds_elems() { return 2 * 16 * MF * (decode_kc<MF>() + 8); }

// One decode-shaped tile: item `it` (rows it.row(0..rows), output columns
// it.chunk * 64 * NFC + [0, 64 * NFC)) of expert it.expert, K in chunks of
// decode_kc<MF>().  All kThreads threads call it; `As0` is decode_lds_elems<MF>()
// bf16 of LDS, free on entry.
template <int MF, int NFC, int PHASE, bool PK = false, bool CMB = false>
__device__ __forceinline__ void decode_tile(const uint16_t* __restrict__ A, const int* __restrict__ arows, int n_x,
                                            int K, const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
                                            int Ncols, const Item& it, uint16_t* __restrict__ out, uint16_t* As0,
                                            const CombineArgs& cmb) {
  constexpr int NF = PHASE == 1 ? 2 * NFC : NFC;
  constexpr int BN = kWaves * 16 * NFC;
  constexpr int BM = 16 * MF;
  constexpr int kDecodeKC = decode_kc<MF>();
  constexpr int kDecodeStride = kDecodeKC + 8;             // bf16 per staged A row (pad 16 B)
  constexpr int U = kDecodeKC / 32;
  constexpr int VPR = kDecodeKC / 8;                       // uint4 per staged row
  constexpr int APT = (BM * VPR + kThreads - 1) / kThreads; // uint4 staged per thread
  auto As = [&](int buf) { return As0 + buf * (BM * kDecodeStride); };
  const int rows = it.rows, e = it.expert;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int l16 = lane & 15, q = lane >> 4;
  const int col0 = it.chunk * BN + wave * 16 * NFC;
  const size_t wstride = static_cast<size_t>(Ncols) * K;
  const int nchunks = (K + kDecodeKC - 1) / kDecodeKC;

  const uint16_t* bp[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int n = min(col0 + (j % NFC) * 16 + l16, Ncols - 1);
    const uint16_t* W = (PHASE == 1 && j >= NFC) ? W1 : W0;
    bp[j] = PK ? W + static_cast<size_t>(e) * wstride + static_cast<size_t>(n / 16) * (K / 32) * 512 + lane * 8
               : W + static_cast<size_t>(e) * wstride + static_cast<size_t>(n) * K + 8 * q;
  }

  // A staging: thread handles uint4 slots idx = tid + s*256 of the chunk
  uint4 stage[APT];
  const uint16_t* arow[APT];
#pragma unroll
  for (int s = 0; s < APT; ++s) {
    const int idx = threadIdx.x + s * kThreads;
    const int r = idx / VPR;
    arow[s] = (idx < BM * VPR && r < rows) ? A + a_row(arows, n_x, it.row(r)) * K : nullptr;
  }
  auto load_a = [&](int c) {
#pragma unroll
    for (int s = 0; s < APT; ++s) {
      const int kv = (threadIdx.x + s * kThreads) % VPR;
      const int k = c * kDecodeKC + kv * 8;
      stage[s] = make_uint4(0, 0, 0, 0);
      if (arow[s] && k < K) stage[s] = *reinterpret_cast<const uint4*>(arow[s] + k);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int s = 0; s < APT; ++s) {
      const int idx = threadIdx.x + s * kThreads;
      if (idx < BM * VPR)
        *reinterpret_cast<uint4*>(As(buf) + (idx / VPR) * kDecodeStride + (idx % VPR) * 8) = stage[s];
    }
  };

  f32x4 acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // weight loads of chunk c (zero past K; a lane's 8 values are all in range or
  // all out)
  auto load_b = [&](uint4 (&b)[U][NF], int c) {
    const int kc = c * kDecodeKC;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = kc + 32 * u + 8 * q;
#pragma unroll
      for (int j = 0; j < NF; ++j)
        b[u][j] = kk < K ? *reinterpret_cast<const uint4*>(bp[j] + (PK ? (kc + 32 * u) * 16 : kc + 32 * u))
                         : make_uint4(0, 0, 0, 0);
    }
  };
  auto mma = [&](const uint4 (&b)[U][NF], const uint16_t* as) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      bf16x8 af[MF];
#pragma unroll
      for (int i = 0; i < MF; ++i)
        af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&as[(16 * i + l16) * kDecodeStride + 32 * u + 8 * q]));
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b[u][j]), af[i], acc[i][j], 0, 0, 0);
    }
  };

  load_a(0);
  store_a(0);
  for (int c = 0; c < nchunks; ++c) {
    uint4 b[U][NF];
    load_b(b, c);
    const bool more = c + 1 < nchunks;
    if (more) load_a(c + 1);
    __syncthreads();                         // chunk c of A is in As[c & 1]
    mma(b, As(c & 1));
    if (more) store_a((c + 1) & 1);          // that buffer was last read before this barrier
  }

  // The MFMA computes (weight rows) x (token rows)^T: in each 16x16 block a
  // lane holds token row l16 and output columns 4q..4q+3, stored as one
  // 8-byte write (Ncols % 8 == 0, so the four columns are all in range or all
  // out).
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const int m = 16 * i + l16;
    if (m >= rows) continue;
    uint16_t* orow = out + static_cast<size_t>(it.row(m)) * Ncols;
#pragma unroll
    for (int j = 0; j < NFC; ++j) {
      const int n = col0 + j * 16 + 4 * q;
      if (n >= Ncols) continue;
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = PHASE == 1 ? silu_mul(acc[i][j][t], acc[i][NFC + j][t]) : acc[i][j][t];
      if constexpr (CMB)
        combine_add4(cmb, it.row(m), Ncols, n, v);
      else
        store4<false>(orow + n, v[0], v[1], v[2], v[3]);
    }
  }
}

template <int MF, int NFC, int PHASE, bool PK = false, bool CMB = false>
__global__ __launch_bounds__(kThreads, MF <= 2 ? kDecodeWavesPerSimd : 2) void ffn_decode_bf16(
    const uint16_t* __restrict__ A, int K, const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
    int Ncols, PlanArgs plan, uint16_t* __restrict__ out, CombineArgs cmb) {
  __shared__ __attribute__((aligned(16))) uint16_t As[decode_lds_elems<MF>()];
  clear_span(plan);
  const int nch = (Ncols + kWaves * 16 * NFC - 1) / (kWaves * 16 * NFC);
  const Item it = block_find_item(plan, nch);
  if (it.rows == 0) return;
  decode_tile<MF, NFC, PHASE, PK, CMB>(A, plan.arows, plan.n_x, K, W0, W1, Ncols, it, out, As, cmb);
}

// ---- decode-sized tiles of one 16-row slab: K split over the waves ----------------
// For the smallest groups (tiles of <= 16 rows, i.e. an average group of at
// most 8 rows) an item is (m-tile, 16*NFC columns) and the block's four waves
// split K into quarters: each streams its quarter of every weight row of the
// item.  A block then moves a quarter of the bytes the kernel above moves per
// item, and there are four times as many items, so the dispatcher keeps
// refilling CUs whose blocks finish early.  On MI355X the blocks resident on
// one CU are served very unevenly (the oldest first); with one round of large
// items the last block on each CU streams alone at the end.  A plain streaming
// kernel of the OLMoE shape moves 537 MB + 268 MB in 134 us with quarter-K
// items against 148 us with whole-K items.  The token rows cost more here (each
// item reads its rows' K range straight into registers, not shared through LDS
// by 64 columns), which is why larger tiles keep the kernel above: at 16 to 32
// rows per tile the extra token-row loads cost more than the balance gains.
//   * B (weight rows) and A (token rows): a lane loads 16 bytes of one row per
//     K-step straight into the v_mfma_f32_16x16x32_bf16 operands; all loads of a
//     batch of U K-steps go out before its first MFMA.  Tile rows past the
//     item's last row read that last row again; their outputs are not stored.
//   * The row-list entries are loaded first and used only after the first
//     batch's weight loads are out, so that round trip overlaps the weights'.
//   * A last partial batch (K not a multiple of 4*32*U) zeroes what lies past
//     the wave's K range.
//   * The waves add their partial sums through LDS; each stores a share of the
//     item's 16x16 output blocks (SwiGLU applied in phase 1).
template <int NFC, int PHASE, bool PK = false, bool CMB = false>
__global__ __launch_bounds__(kThreads, kDecodeWavesPerSimd) void ffn_decode_splitk_bf16(
    const uint16_t* __restrict__ A, int K, const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
    int Ncols, PlanArgs plan, uint16_t* __restrict__ out, CombineArgs cmb) {
  constexpr int NF = PHASE == 1 ? 2 * NFC : NFC;
  constexpr int BN = 16 * NFC;
  constexpr int U = 4;
  constexpr int KB = 32 * U;                          // K per batch
  __shared__ f32x4 part[kWaves][NF][kWave];           // partial sums, 16 B per lane per block

  clear_span(plan);
  const int nch = (Ncols + BN - 1) / BN;
  const Item it = block_find_item(plan, nch);
  if (it.rows == 0) return;
  const int rows = it.rows, e = it.expert;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  const int l16 = lane & 15, q = lane >> 4;
  const int col0 = it.chunk * BN;
  const size_t wstride = static_cast<size_t>(Ncols) * K;
  // this wave's K range: a quarter of K rounded up to whole K-steps
  const int kq = (K + kWaves * 32 - 1) / (kWaves * 32) * 32;
  const int k0 = min(K, wave * kq), k1 = min(K, k0 + kq);

  const uint16_t* bp[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int n = min(col0 + (j % NFC) * 16 + l16, Ncols - 1);
    const uint16_t* W = (PHASE == 1 && j >= NFC) ? W1 : W0;
    bp[j] = PK ? W + static_cast<size_t>(e) * wstride + static_cast<size_t>(n / 16) * (K / 32) * 512 + lane * 8
               : W + static_cast<size_t>(e) * wstride + static_cast<size_t>(n) * K + 8 * q;
  }
  f32x4 acc[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Batch of U K-steps from kc.  MASK: zero what lies at or past k1 (a lane's
  // 8 values are all below k1 or all at or past it: K and k1 are multiples of
  // 8), reading the row's first 16 bytes instead.
  const uint16_t* ap = nullptr;
  uint4 b[U][NF], a[U];
  auto koff = [&](auto mask, int kk) { return (!decltype(mask)::value || kk + 8 * q < k1) ? kk : -8 * q; };
  auto load_b = [&](auto mask, int kc) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ko = koff(mask, kc + 32 * u);
#pragma unroll
      for (int j = 0; j < NF; ++j) b[u][j] = *reinterpret_cast<const uint4*>(bp[j] + (PK ? ko * 16 : ko));
    }
  };
  auto load_a = [&](auto mask, int kc) {
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = *reinterpret_cast<const uint4*>(ap + koff(mask, kc + 32 * u));
  };
  auto mma = [&](auto mask, int kc) {
    if constexpr (decltype(mask)::value) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (kc + 32 * u + 8 * q >= k1) {
#pragma unroll
          for (int j = 0; j < NF; ++j) b[u][j] = make_uint4(0, 0, 0, 0);
          a[u] = make_uint4(0, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NF; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b[u][j]),
                                                         __builtin_bit_cast(bf16x8, a[u]), acc[j], 0, 0, 0);
  };
  // The sched_barriers keep every load of a batch ahead of its first MFMA
  // (left alone, the scheduler interleaves them and waits after the first
  // few).  The first batch always takes the masked form: with a branch
  // between the row-list load and its use the compiler hoists the use and
  // waits for the list before any weight load.
  if (k0 < k1) {
    const int rn[1] = {it.row(min(l16, rows - 1))};
    int raw[1];
    a_rows_raw(plan.arows, plan.offs, rn, raw);
    __builtin_amdgcn_sched_barrier(0);
    load_b(std::true_type{}, k0);
    __builtin_amdgcn_sched_barrier(0);
    ap = A + a_row_of(plan.arows, plan.n_x, rn[0], raw[0]) * K + 8 * q;
    load_a(std::true_type{}, k0);
    __builtin_amdgcn_sched_barrier(0);
    mma(std::true_type{}, k0);
    int kc = min(k0 + KB, k1);
    for (; kc + KB <= k1; kc += KB) {
      load_b(std::false_type{}, kc);
      load_a(std::false_type{}, kc);
      __builtin_amdgcn_sched_barrier(0);
      mma(std::false_type{}, kc);
    }
    if (kc < k1) {
      load_b(std::true_type{}, kc);
      load_a(std::true_type{}, kc);
      __builtin_amdgcn_sched_barrier(0);
      mma(std::true_type{}, kc);
    }
  }

  // Sum the four waves' partials.  The MFMA computes (weight rows) x (token
  // rows)^T: in each 16x16 block a lane holds token row l16 and output columns
  // 4q..4q+3, stored as one 8-byte write (Ncols % 8 == 0, so the four columns
  // are all in range or all out).  Output block j goes to wave j % 4.
#pragma unroll
  for (int j = 0; j < NF; ++j) part[wave][j][lane] = acc[j];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NFC; ++j) {
    if (j % kWaves != wave) continue;
    const int n = col0 + j * 16 + 4 * q;
    if (l16 >= rows || n >= Ncols) continue;
    f32x4 g = part[0][j][lane], u = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 1; w < kWaves; ++w) g += part[w][j][lane];
    if constexpr (PHASE == 1) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) u += part[w][NFC + j][lane];
    }
    float v[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = PHASE == 1 ? silu_mul(g[t], u[t]) : g[t];
    if constexpr (CMB) {
      combine_add4(cmb, it.row(l16), Ncols, n, v);
    } else {
      uint16_t* orow = out + static_cast<size_t>(it.row(l16)) * Ncols;
      *reinterpret_cast<uint2*>(orow + n) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
  }
}

// The fused combine's last step: y = bf16(y32), eight values per thread.
__global__ void ffn_combine_finalize(const float* __restrict__ y32, uint16_t* __restrict__ y, int n8) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const float4 a = reinterpret_cast<const float4*>(y32)[2 * i], b = reinterpret_cast<const float4*>(y32)[2 * i + 1];
  reinterpret_cast<uint4*>(y)[i] = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                                              pack_bf16x2(b.z, b.w));
}

// ---- decode-sized tiles with FP8 weights ---------------------------------------
// ExpertPlex page, "Experimental results" (models table): GLM-5.1-FP8 serves its
// experts in FP8.  Weights are OCP E4M3 codes with one fp32 scale per weight
// row (per output feature); token rows and the SwiGLU product stay bf16.  The
// structure is ffn_decode_bf16's with eight waves per block and twice the K
// per chunk:
//   * a lane loads 16 bytes = 16 weights of one row (each row still streams in
//     64-byte runs per instruction) and converts them with
//     v_cvt_scalef32_pk_bf16_fp8 (exact: every E4M3 value is a bf16 value)
//     into the B operands of two v_mfma_f32_16x16x32_bf16 K-steps: in K-step h
//     lane (l16, q) holds weights kk + 16 q + 8 h .. + 7 and reads the same
//     eight values of its token row from LDS (the MFMA sums over its 32 K
//     values, so any split of the 64 values between the two steps works as
//     long as both operands use it);
//   * a chunk is 512 K values for 16-row tiles, so a wave keeps 16 KiB of
//     weights in flight as in the bf16 kernel; 384 for 32-row tiles (at 512
//     their accumulators and staging spill registers to scratch, which cost
//     a sixth of the OLMoE-shaped call) and 256 for 64-row tiles (LDS); the
//     chunk's token rows are staged through LDS, double buffered, and shared
//     by the eight waves (two blocks per CU fit in LDS);
//   * the row scale multiplies the fp32 accumulator before SwiGLU or the store.
constexpr int kThreads8 = 512;
constexpr int kWaves8 = kThreads8 / kWave;
template <int MF>
constexpr int fp8_kc() { return MF == 1 ? 512 : MF == 2 ? 384 : 256; }

// Eight E4M3 codes (two 32-bit words, lowest byte first) as eight bf16 values.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int MF, int NFC, int PHASE, bool PK = false>
__global__ __launch_bounds__(kThreads8, 4) void ffn_decode_fp8w(
    const uint16_t* __restrict__ A, int K, const uint8_t* __restrict__ W0, const uint8_t* __restrict__ W1,
    const float* __restrict__ S0, const float* __restrict__ S1, int Ncols, PlanArgs plan,
    uint16_t* __restrict__ out) {
  constexpr int NF = PHASE == 1 ? 2 * NFC : NFC;
  constexpr int BN = kWaves8 * 16 * NFC;
  constexpr int BM = 16 * MF;
  constexpr int KC = fp8_kc<MF>();
  constexpr int kStride = KC + 8;                           // bf16 per staged A row (pad 16 B)
  constexpr int U = KC / 64;                                // 16-byte weight loads per row per chunk
  constexpr int VPR = KC / 8;                               // uint4 per staged A row
  constexpr int APT = (BM * VPR + kThreads8 - 1) / kThreads8;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kStride];

  const int nch = (Ncols + BN - 1) / BN;
  const Item it = block_find_item<kThreads8>(plan, nch);
  if (it.rows == 0) return;
  const int rows = it.rows, e = it.expert;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int l16 = lane & 15, q = lane >> 4;
  const int col0 = it.chunk * BN + wave * 16 * NFC;
  const int nchunks = (K + KC - 1) / KC;

  const uint8_t* bp[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int n = min(col0 + (j % NFC) * 16 + l16, Ncols - 1);
    const uint8_t* W = (PHASE == 1 && j >= NFC) ? W1 : W0;
    // packed: blocks of 16 rows x 64 codes (1 KiB), lane 16 q + l16 at byte 16 * lane
    bp[j] = W + fp8_code_offset(e, n, K, Ncols, lane, 0, PK);
  }

  // token rows of a chunk: thread handles uint4 slots idx = tid + s * 512
  uint4 stage[APT];
  const uint16_t* arow[APT];
#pragma unroll
  for (int s = 0; s < APT; ++s) {
    const int idx = threadIdx.x + s * kThreads8;
    const int r = idx / VPR;
    arow[s] = (idx < BM * VPR && r < rows) ? A + a_row(plan.arows, plan.n_x, it.row(r)) * K : nullptr;
  }
  auto load_a = [&](int c) {
#pragma unroll
    for (int s = 0; s < APT; ++s) {
      const int kv = (threadIdx.x + s * kThreads8) % VPR;
      const int k = c * KC + kv * 8;
      stage[s] = make_uint4(0, 0, 0, 0);
      if (arow[s] && k < K) stage[s] = *reinterpret_cast<const uint4*>(arow[s] + k);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int s = 0; s < APT; ++s) {
      const int idx = threadIdx.x + s * kThreads8;
      if (idx < BM * VPR)
        *reinterpret_cast<uint4*>(&As[buf][(idx / VPR) * kStride + (idx % VPR) * 8]) = stage[s];
    }
  };

  f32x4 acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // weight loads of chunk c (zero past K: K % 16 == 0, so a lane's 16 codes
  // are all in range or all out)
  auto load_b = [&](uint4 (&b)[U][NF], int c) {
    const int kc = c * KC;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = kc + 64 * u + 16 * q;
#pragma unroll
      for (int j = 0; j < NF; ++j)
        b[u][j] = kk < K ? *reinterpret_cast<const uint4*>(bp[j] + fp8_code_step(kc + 64 * u, PK))
                         : make_uint4(0, 0, 0, 0);
    }
  };
  auto mma = [&](const uint4 (&b)[U][NF], const uint16_t* as) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 af[MF];
#pragma unroll
        for (int i = 0; i < MF; ++i)
          af[i] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const uint4*>(&as[(16 * i + l16) * kStride + 64 * u + 16 * q + 8 * h]));
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          const bf16x8 bw = h == 0 ? fp8x8_to_bf16(b[u][j].x, b[u][j].y) : fp8x8_to_bf16(b[u][j].z, b[u][j].w);
#pragma unroll
          for (int i = 0; i < MF; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw, af[i], acc[i][j], 0, 0, 0);
        }
      }
  };

  load_a(0);
  store_a(0);
  for (int c = 0; c < nchunks; ++c) {
    uint4 b[U][NF];
    load_b(b, c);
    const bool more = c + 1 < nchunks;
    if (more) load_a(c + 1);
    __syncthreads();                           // chunk c of A is in As[c & 1]
    mma(b, As[c & 1]);
    if (more) store_a((c + 1) & 1);            // that buffer was last read before this barrier
  }

  // In each 16x16 block a lane holds token row l16 and output columns
  // 4q..4q+3 (one 8-byte store; Ncols % 16 == 0, so all four are in range or
  // all out); the four columns' scales load as one float4.
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const int m = 16 * i + l16;
    if (m >= rows) continue;
    uint16_t* orow = out + static_cast<size_t>(it.row(m)) * Ncols;
#pragma unroll
    for (int j = 0; j < NFC; ++j) {
      const int n = col0 + j * 16 + 4 * q;
      if (n >= Ncols) continue;
      const size_t so = static_cast<size_t>(e) * Ncols + n;
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(S0 + so);
      float v[4];
      if constexpr (PHASE == 1) {
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(S1 + so);
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = silu_mul(acc[i][j][t] * s0[t], acc[i][NFC + j][t] * s1[t]);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = acc[i][j][t] * s0[t];
      }
      *reinterpret_cast<uint2*>(orow + n) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
  }
}

// ---- prefill-sized tiles: LDS-tiled GEMM on v_mfma_f32_32x32x16_bf16 ------------
// Block tile: BM token rows x BN weight rows (phase 1: BN/2 gate rows then the
// matching BN/2 up rows -> BN/2 SwiGLU columns; phase 2: BN down rows), K in
// steps of kGemmBK = 32.
//   * Operands go HBM -> LDS directly (global_load_lds_dwordx4: each lane's 16
//     bytes land at LDS base + 16*lane, no VGPR staging, no LDS store
//     instructions), through a ring of STAGES K-step buffers: STAGES-1 K-steps
//     are in flight while one is multiplied; one barrier per K-step.
//   * LDS rows are 64 bytes (four 16-byte chunks) with no padding; chunk c of
//     row r sits at slot c ^ swz(r), swz(r) = ((r >> 1) ^ (r >> 2)) & 3.  An
//     MFMA operand read (16 lanes: 16 consecutive rows, one chunk) then hits
//     16 distinct 4-bank groups, and so does any 8-lane group.  The DMA side
//     writes 1 KiB contiguously per instruction and applies the swizzle by
//     choosing which global chunk each lane fetches.
//   * WM x WN waves, each (32*MI) x (32*NJ) as MI x NJ blocks of 32x32
//     (phase 1: NJ/2 gate blocks and the same columns' NJ/2 up blocks, so
//     SwiGLU needs no exchange).  The weight rows are the MFMA's first operand,
//     so the accumulators come out transposed and each lane stores four
//     consecutive output columns at once.
// Two shapes: 128 x 256 with four waves and two blocks per CU (any group
// sizes), and 256 x 256 with eight waves and one block per CU, which moves a
// third fewer bytes per flop from L2 and keeps four K-steps in flight, for
// batches whose groups average at least kGemmLargeMinAvg rows.
// The K extent must be a multiple of kGemmBK (checked by the host).
constexpr int kGemmBK = 32;
constexpr int kGemmRowBytes = kGemmBK * 2;
constexpr int kEpiPitch = 80;                 // bytes per row of a wave's 32x32 bf16 epilogue block (64 + 16 pad)
constexpr int kEpiBytes = 32 * kEpiPitch;     // per wave

// F8: the weights are E4M3 codes (one byte each) pre-packed by
// pack_fp8_codes, so a K-step moves 32 bytes per weight row instead of 64.
template <int MI_, int NJ_, int WM_, int WN_, int STAGES_, int BPC_, bool F8_ = false>
struct GemmCfg {
  static constexpr int MI = MI_, NJ = NJ_, WM = WM_, WN = WN_, STAGES = STAGES_, BLOCKS_PER_CU = BPC_;
  static constexpr bool F8 = F8_;
  static constexpr int NW = WM * WN, NT = kWave * NW;
  static constexpr int BM = 32 * MI * WM, BN = 32 * NJ * WN;
  static constexpr int A_BYTES = BM * kGemmRowBytes, B_BYTES = BN * (F8 ? kGemmBK : kGemmRowBytes);
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int RING = STAGES * STAGE;               // LDS bytes of the operand ring
  static constexpr int ADMA = BM / 16 / NW;                 // 1 KiB DMA instructions per wave per K-step
  static constexpr int BDMA = B_BYTES / 1024 / NW;
};
using GemmSmall = GemmCfg<2, 4, 2, 2, 3, 2>;   // 128 x 256
using GemmLarge = GemmCfg<2, 4, 4, 2, 4, 1>;   // 256 x 256
// 256 x 256 on FP8 codes: a stage is 24 KiB, so five fit (four K-steps in flight)
using GemmLargeF8 = GemmCfg<2, 4, 4, 2, 5, 1, true>;
// 128 x 256 on FP8 codes: a stage is 16 KiB, four per block, two blocks per CU
using GemmSmallF8 = GemmCfg<2, 4, 2, 2, 4, 2, true>;
constexpr int kGemmLargeMinAvg = 256;

__device__ __forceinline__ int gemm_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// 16 bytes per lane from global memory to LDS byte address lds + 16*lane.
// Issued as inline assembly so that the compiler does not treat every later
// LDS read as dependent on it (it would wait for all loads in flight); the
// kernel orders it with explicit vmcnt waits and barriers instead.
__device__ __forceinline__ void dma_b128(const void* g, uint32_t lds) {
  // M0 carries the wave-uniform LDS base; one wait state between writing M0
  // and an LDS-DMA load is required
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(lds) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
}

// Wait until at most `ahead` K-steps of PER loads each are still in flight,
// then barrier (ahead <= MAXA, wave-uniform).
template <int PER, int MAXA>
__device__ __forceinline__ void wait_ahead_barrier(int ahead) {
  if constexpr (MAXA == 0) {
    wait_vm_barrier<0>();
  } else {
    if (ahead >= MAXA)
      wait_vm_barrier<MAXA * PER>();
    else
      wait_ahead_barrier<PER, MAXA - 1>(ahead);
  }
}

// Pieces of a tile, shared by the one-tile and the persistent kernels.  All
// threads of the block call them.
//
// TileLoader: DMA sources of one tile.  Instruction q of a wave fills tile
// rows 16 (wave + NW q) .. +15; lane -> row + lane / 4, slot lane % 4, fetching
// chunk slot ^ swz(row).  Rows past the tile's valid rows / columns read a
// valid row instead (their results are never stored).
// PKB: the weights are pre-packed (pack_weights: blocks of 16 rows x 32 K,
// 1 KiB each, (row block, K block) order; inside a block lane 16 q + r's 16
// bytes are W[r][8q .. 8q+7]).  A K-step of 16 weight rows is then one
// contiguous KiB, which one DMA instruction copies as is: in LDS the block's
// row r, chunk c sits at byte c * 256 + r * 16 (no swizzle needed: a 16-lane
// group of an operand read covers 256 contiguous bytes).
// C::F8: the weights are E4M3 codes packed by pack_fp8_codes (blocks of 16
// rows x 64 codes, 1 KiB, (row block, K block) order; inside a block codes
// [16 kq, 16 kq + 16) of row r at byte (16 kq + r) * 16).  A K-step of 32
// codes is half a block (kq = 2 (kt % 2) + 0, 1: 512 contiguous bytes), so an
// instruction copies the halves of two row blocks: lanes 0-31 rows rb..rb+15,
// lanes 32-63 rows rb+16..rb+31.  In LDS the instruction's 1 KiB holds, per
// row block b (512 bytes each), codes [16 s, 16 s + 16) of row r at byte
// b * 512 + (16 s + r) * 16.
template <int PHASE, class C, bool PKB = false>
struct TileLoader {
  const uint16_t* asrc[C::ADMA];
  const uint16_t* bsrc[C::BDMA];
  const uint8_t* bsrc8[C::BDMA];
  const float* ssrc;   // C::F8: this lane's 16 bytes of the tile's weight-row scales
  int na;   // this wave's A instructions whose first row is valid (wave-uniform): 0..ADMA

  // A DMA instructions wave `wave` issues per K-step for a tile of `rows` rows
  __device__ __forceinline__ static int a_issued(int wave, int rows) {
    int n = 0;
#pragma unroll
    for (int q = 0; q < C::ADMA; ++q) n += 16 * (wave + C::NW * q) < rows ? 1 : 0;
    return n;
  }

  __device__ __forceinline__ void init(const uint16_t* __restrict__ A, const int* __restrict__ arows, int n_x, int K,
                                       const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1, int Ncols,
                                       const Item& it, const float* __restrict__ S0 = nullptr,
                                       const float* __restrict__ S1 = nullptr) {
    constexpr int OUTC = PHASE == 1 ? C::BN / 2 : C::BN;
    const int wave = threadIdx.x >> 6, lane = lane_id(), dr = lane >> 2;
    const int n0 = it.chunk * OUTC;
    const size_t eoff = static_cast<size_t>(it.expert) * Ncols * K;
    na = __builtin_amdgcn_readfirstlane(a_issued(wave, it.rows));
    int rn[C::ADMA];
    size_t ar[C::ADMA];
#pragma unroll
    for (int q = 0; q < C::ADMA; ++q) rn[q] = it.row(min(16 * (wave + C::NW * q) + dr, it.rows - 1));
    a_rows(arows, n_x, rn, ar);
#pragma unroll
    for (int q = 0; q < C::ADMA; ++q) {
      const int r = 16 * (wave + C::NW * q) + dr;
      asrc[q] = A + ar[q] * K + 8 * ((lane & 3) ^ gemm_swz(r));
    }
#pragma unroll
    for (int q = 0; q < C::BDMA; ++q) {
      if constexpr (C::F8) {
        // W0 / W1 hold bytes here (E4M3 codes); 32 tile rows per instruction
        const int rb = 32 * (wave + C::NW * q);
        int nb = n0 + rb + 16 * (lane >> 5);
        const uint8_t* W = reinterpret_cast<const uint8_t*>(W0);
        if (PHASE == 1 && rb >= OUTC) {
          nb -= OUTC;
          W = reinterpret_cast<const uint8_t*>(W1);
        }
        nb = min(nb, Ncols - 16);                        // blocks past the rows are read but never stored
        bsrc8[q] = W + eoff + static_cast<size_t>(nb / 16) * (K / 64) * 1024 + (lane & 31) * 16;
        // scales of the tile's weight rows, 1 KiB: phase 1 lanes 0-31 the 128
        // gate rows, lanes 32-63 the 128 up rows; phase 2 the 256 down rows
        // (columns past Ncols read the last four, never used)
        const int c = PHASE == 1 ? 4 * (lane & 31) : 4 * lane;
        const float* S = (PHASE == 1 && lane >= 32) ? S1 : S0;
        ssrc = S + static_cast<size_t>(it.expert) * Ncols + min(n0 + c, Ncols - 4);
      } else if constexpr (PKB) {
        const int rb = 16 * (wave + C::NW * q);         // first tile row of this instruction
        int nb = n0 + rb;
        const uint16_t* W = W0;
        if (PHASE == 1 && rb >= OUTC) {
          nb -= OUTC;
          W = W1;
        }
        nb = min(nb, Ncols - 16);                        // blocks past the rows are read but never stored
        bsrc[q] = W + eoff + static_cast<size_t>(nb / 16) * (K / 32) * 512 + lane * 8;
      } else {
        const int r = 16 * (wave + C::NW * q) + dr;
        int n = n0 + r;
        const uint16_t* W = W0;
        if (PHASE == 1 && r >= OUTC) {
          n -= OUTC;
          W = W1;
        }
        bsrc[q] = W + eoff + static_cast<size_t>(min(n, Ncols - 1)) * K + 8 * ((lane & 3) ^ gemm_swz(r));
      }
    }
  }

  // C::F8: the tile's scales into 1 KiB of LDS at byte address `dst` (one
  // instruction; the caller's waits on later K-steps cover it).
  __device__ __forceinline__ void issue_scales(uint32_t dst) const { dma_b128(ssrc, dst); }

  // K-step kt of this tile into ring slot `slot` (lds0: LDS byte address of the ring).
  // With skip_a, A instructions whose rows all lie past the tile's rows are
  // not issued (their LDS rows keep stale data, whose results are never
  // stored); the wave then has na + BDMA loads per step in flight.
  template <bool skip_a = false>
  __device__ __forceinline__ void issue(int kt, int slot, uint32_t lds0) const {
    const uint32_t st = lds0 + slot * C::STAGE + (threadIdx.x >> 6) * 1024;
    const int k = kt * kGemmBK;
#pragma unroll
    for (int q = 0; q < C::ADMA; ++q)
      if (!skip_a || q < na) dma_b128(asrc[q] + k, st + q * C::NW * 1024);
#pragma unroll
    for (int q = 0; q < C::BDMA; ++q) {
      if constexpr (C::F8)
        dma_b128(bsrc8[q] + (kt >> 1) * 1024 + (kt & 1) * 512, st + C::A_BYTES + q * C::NW * 1024);
      else
        dma_b128(bsrc[q] + (PKB ? kt * 512 : k), st + C::A_BYTES + q * C::NW * 1024);
    }
  }
};

// TileMath: the wave's MFMA work on one ring slot, and the epilogue.
// MFMA operand rows of this wave: A rows 32 (wm + WM i) + l32 (the waves'
// 32-row slabs interleave, so a partial tile's valid slabs spread over all
// waves, and a wave skips the MFMAs and LDS reads of its slabs that lie wholly
// past the tile's valid rows); weight rows:
// phase 2 (BN/WN) wn + 32 j + l32; phase 1 gate block j < NJ/2 at
// (BN/2/WN) wn + 32 j + l32, up block j >= NJ/2 at BN/2 + (BN/2/WN) wn +
// 32 (j - NJ/2) + l32.  Every block starts at a multiple of 32 rows, so the
// swizzle depends on l32 only.
template <int V>
struct Int {
  static constexpr int value = V;
};

template <int PHASE, class C, bool PKB = false>
struct TileMath {
  static constexpr int MI = C::MI, NJ = C::NJ, WM = C::WM, WN = C::WN, BN = C::BN;
  static_assert(PHASE == 2 || NJ % 2 == 0, "phase 1 pairs gate and up blocks");
  static_assert(MI == 1 || MI == 2, "kstep dispatches on 0, 1 or MI valid slabs");
  static_assert(C::ADMA >= 1 && C::BDMA >= 1, "tile too small for its waves");
  static_assert(C::STAGES >= 2, "the ring needs two buffers");
  int boff[NJ];
  int aoff, loff[2], loffb[2];
  int wm, wn, l32, hk;
  int nv;                 // this wave's slabs holding valid rows (wave-uniform)
  f32x16 acc[MI][NJ];

  __device__ __forceinline__ void init() {
    const int wave = threadIdx.x >> 6, lane = lane_id();
    wm = wave / WN;
    wn = wave % WN;
    l32 = lane & 31;
    hk = lane >> 5;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int rb = PHASE == 1 ? (j < NJ / 2 ? 0 : BN / 2) + (BN / 2 / WN) * wn + 32 * (j % (NJ / 2))
                                : (BN / WN) * wn + 32 * j;
      boff[j] = C::A_BYTES + (C::F8 ? (rb / 32) * 1024 : rb * kGemmRowBytes);
    }
    aoff = 32 * wm * kGemmRowBytes;
    nv = MI;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      loff[s] = l32 * kGemmRowBytes + 16 * ((2 * s + hk) ^ gemm_swz(l32));
      loffb[s] = C::F8 ? (l32 / 16) * 512 + (16 * s + l32 % 16) * 16 + 8 * hk
                 : PKB ? (l32 / 16) * 1024 + (2 * s + hk) * 256 + (l32 % 16) * 16 : loff[s];
    }
  }

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  // valid rows of the next tile: slab i of this wave holds rows
  // 32 (wm + WM i) .. +31, valid if its first row is
  __device__ __forceinline__ void set_rows(int rows) {
    const int slabs = (rows + 31) >> 5;
    nv = __builtin_amdgcn_readfirstlane(min(MI, max(0, (slabs - wm + WM - 1) / WM)));
  }

  // FP8 weights: multiply each accumulator by its weight row's scale, from
  // the tile's scales in LDS (TileLoader::issue_scales: phase 1 gate rows at
  // [0, BN/2) and up rows at [BN/2, BN), phase 2 rows at [0, BN)), before the
  // epilogue's SwiGLU or store.
  __device__ __forceinline__ void apply_scales(const float* sc) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c0 = PHASE == 1 ? (j < NJ / 2 ? 0 : BN / 2) + (BN / 2 / WN) * wn + 32 * (j % (NJ / 2)) + 4 * hk
                                : (BN / WN) * wn + 32 * j + 4 * hk;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(sc + c0 + 8 * q);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          acc[i][j][4 * q + 0] *= v.x;
          acc[i][j][4 * q + 1] *= v.y;
          acc[i][j][4 * q + 2] *= v.z;
          acc[i][j][4 * q + 3] *= v.w;
        }
      }
    }
  }

  template <int NV>
  __device__ __forceinline__ void kstep_n(const uint8_t* st) {
    if constexpr (NV == 0) return;                // no valid rows: nothing to read or multiply
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 af[NV > 0 ? NV : 1], bf[NJ];
#pragma unroll
      for (int i = 0; i < NV; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(st + aoff + 32 * WM * i * kGemmRowBytes + loff[s]);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if constexpr (C::F8) {
          // eight codes of this lane's weight row, converted exactly to bf16
          const uint2 c = *reinterpret_cast<const uint2*>(st + boff[j] + loffb[s]);
          bf[j] = fp8x8_to_bf16(c.x, c.y);
        } else {
          bf[j] = *reinterpret_cast<const bf16x8*>(st + boff[j] + loffb[s]);
        }
      }
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
    }
  }

  // Runs body(Int<NV>) with NV = nv as a compile-time constant, so that the
  // K loop inside body has no per-step branch (a branch around the MFMAs of
  // every step makes the compiler copy and spill the accumulators).
  template <class Body>
  __device__ __forceinline__ void with_nv(Body&& body) {
    if (nv == MI) {
      body(Int<MI>{});
    } else if constexpr (MI == 2) {
      if (nv == 1) body(Int<1>{});
      else body(Int<0>{});
    } else {
      body(Int<0>{});
    }
  }

  // The MFMA computes (weight rows) x (token rows)^T, so in each 32x32
  // accumulator block a lane holds token row l32 and output columns
  // 8 (r/4) + 4 hk + r % 4: four consecutive columns per r/4, stored as one
  // 8-byte write (Ncols is a multiple of 32 on this path).
  template <bool COHERENT = false>
  __device__ __forceinline__ void store(const Item& it, int Ncols, uint16_t* __restrict__ out) const {
    constexpr int OUTC = PHASE == 1 ? BN / 2 : BN;
    const int n0 = it.chunk * OUTC;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = 32 * (wm + WM * i) + l32;
      if (m >= it.rows) continue;
      uint16_t* orow = out + static_cast<size_t>(it.row(m)) * Ncols;
#pragma unroll
      for (int j = 0; j < (PHASE == 1 ? NJ / 2 : NJ); ++j) {
        const int nb = n0 + (PHASE == 1 ? (BN / 2 / WN) * wn : (BN / WN) * wn) + 32 * j + 4 * hk;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nb + 8 * q;
          if (n >= Ncols) continue;
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            v[t] = PHASE == 1 ? silu_mul(acc[i][j][4 * q + t], acc[i][NJ / 2 + j][4 * q + t]) : acc[i][j][4 * q + t];
          store4<COHERENT>(orow + n, v[0], v[1], v[2], v[3]);
        }
      }
    }
  }

  // The same epilogue through a wave-private LDS block of 32 rows x 32
  // columns (pitch kEpiPitch bytes): a lane's four 8-byte pieces go to LDS,
  // and the block leaves as 16-byte stores of 64-byte row segments, two
  // instructions per block instead of four of scattered 8-byte pieces (the
  // store count halves and each instruction covers 16 rows, not 32).
  __device__ __forceinline__ void store_staged(const Item& it, int Ncols, uint16_t* __restrict__ out,
                                               uint8_t* wst) const {
    constexpr int OUTC = PHASE == 1 ? BN / 2 : BN;
    constexpr int NO = PHASE == 1 ? NJ / 2 : NJ;
    const int n0 = it.chunk * OUTC;
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int mb = 32 * (wm + WM * i);
      if (mb >= it.rows) continue;                      // wave-uniform: no valid row in this slab
#pragma unroll
      for (int j = 0; j < NO; ++j) {
        const int cb = n0 + (PHASE == 1 ? (BN / 2 / WN) * wn : (BN / WN) * wn) + 32 * j;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            v[t] = PHASE == 1 ? silu_mul(acc[i][j][4 * q + t], acc[i][NJ / 2 + j][4 * q + t]) : acc[i][j][4 * q + t];
          *reinterpret_cast<uint2*>(wst + l32 * kEpiPitch + (8 * q + 4 * hk) * 2) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = 16 * h + (lane >> 2), c = 8 * (lane & 3);
          const uint4 v = *reinterpret_cast<const uint4*>(wst + r * kEpiPitch + 2 * c);
          if (mb + r < it.rows && cb + c < Ncols)
            *reinterpret_cast<uint4*>(out + static_cast<size_t>(it.row(mb + r)) * Ncols + cb + c) = v;
        }
      }
    }
  }
};

__device__ __forceinline__ uint32_t lds_address(const uint8_t* smem) {
  typedef __attribute__((address_space(3))) const uint8_t lds_byte;
  return (uint32_t)(uintptr_t)(lds_byte*)smem;
}

// One tile: the it.rows sorted rows it.row(0..) of A against output column chunk
// `it.chunk` of expert `it.expert`.  `smem` is the block's operand ring, free
// on entry (no wave still reads it).  C::F8: W0 / W1 hold packed E4M3 codes,
// S0 / S1 their row scales, and `scl` is 1 KiB of LDS for the tile's scales
// (free on entry too).
template <int PHASE, class C, bool COHERENT = false, bool PKB = false>
__device__ __forceinline__ void gemm_tile(const uint16_t* __restrict__ A, const int* __restrict__ arows, int n_x,
                                          int K, const uint16_t* __restrict__ W0,
                                          const uint16_t* __restrict__ W1, int Ncols, const Item& it,
                                          uint16_t* __restrict__ out, uint8_t* smem,
                                          const float* __restrict__ S0 = nullptr,
                                          const float* __restrict__ S1 = nullptr, float* scl = nullptr) {
  constexpr int STAGES = C::STAGES;
  TileLoader<PHASE, C, PKB> ld;
  ld.init(A, arows, n_x, K, W0, W1, Ncols, it, S0, S1);
  TileMath<PHASE, C, PKB> mm;
  mm.init();
  mm.set_rows(it.rows);
  mm.zero();
  const uint32_t lds0 = lds_address(smem);
  const int nk = K / kGemmBK;
  // C::F8: wave 0 loads the tile's scales first; its extra load only makes its
  // waits stricter, and the first K-step's wait and barrier make the scales
  // visible to every wave
  if constexpr (C::F8)
    if ((threadIdx.x >> 6) == 0) ld.issue_scales(lds_address(reinterpret_cast<const uint8_t*>(scl)));
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) ld.template issue<true>(s, s, lds0);
  // a wave issues na + BDMA loads per K-step (na wave-uniform), so its waits
  // count that many per step still in flight
  auto loop = [&](auto nac) {
    constexpr int PER = decltype(nac)::value + C::BDMA;
    mm.with_nv([&](auto nvc) {
      for (int kt = 0; kt < nk; ++kt) {
        // K-step kt's loads are done once only the later steps' remain in flight
        wait_ahead_barrier<PER, STAGES - 2>(min(STAGES - 2, nk - 1 - kt));
        // every wave is past step kt-1, so its buffer can be refilled
        if (kt + STAGES - 1 < nk) ld.template issue<true>(kt + STAGES - 1, (kt + STAGES - 1) % STAGES, lds0);
        mm.template kstep_n<decltype(nvc)::value>(smem + (kt % STAGES) * C::STAGE);
      }
    });
  };
  static_assert(C::ADMA <= 2, "per-wave A instruction counts 0..2");
  if (ld.na == C::ADMA) loop(Int<C::ADMA>{});
  else if (ld.na == 1) loop(Int<1>{});
  else loop(Int<0>{});
  if constexpr (C::F8) mm.apply_scales(scl);
  mm.template store<COHERENT>(it, Ncols, out);
}

// One tile per block, blocks dealt by the hardware (two resident per CU, so
// one block's start-up overlaps the other's work).
template <int PHASE, class C, bool PKB>
__global__ __launch_bounds__(C::NT, C::BLOCKS_PER_CU) void ffn_gemm_bf16(
    const uint16_t* __restrict__ A, int K, const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
    int Ncols, PlanArgs plan, uint16_t* __restrict__ out, const float* __restrict__ S0,
    const float* __restrict__ S1) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::RING];
  __shared__ __attribute__((aligned(16))) float scl[C::F8 ? 256 : 1];
  constexpr int OUTC = PHASE == 1 ? C::BN / 2 : C::BN;
  const Item it = block_find_item<C::NT>(plan, (Ncols + OUTC - 1) / OUTC);
  if (it.rows == 0) return;
  gemm_tile<PHASE, C, false, PKB>(A, plan.arows, plan.n_x, K, W0, W1, Ncols, it, out, smem, S0, S1, scl);
}

// ---- persistent GEMM launch: each block walks a list of tiles ----------------
// Used for the one-block-per-CU large tile, where a block that ended would
// leave its CU idle until the next one started.
// Grid = BLOCKS_PER_CU blocks per CU (a multiple of 8).  Items are ordered as
// for the one-tile kernels (group by group, column chunk by column chunk,
// m-tile by m-tile); XCD x (blocks dealt round-robin) owns the x-th eighth of
// the list and its blocks take that eighth's items in turn.  A block runs its
// items' K-steps as one stream through the ring, so the next tile's first
// K-steps load while the current tile finishes and stores: no per-tile
// prologue bubble, no block launch per tile.
// With C::F8, W0 / W1 point to E4M3 codes packed by pack_fp8_codes and S0 /
// S1 to their row scales ([E+S][Ncols] fp32; S0 for the gate or down rows,
// S1 for the up rows); the scales multiply the accumulators before the
// epilogue.
template <int PHASE, class C, bool PKB>
__global__ __launch_bounds__(C::NT, C::BLOCKS_PER_CU) void ffn_gemm_persistent_bf16(
    const uint16_t* __restrict__ A, int K, const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
    int Ncols, PlanArgs plan, uint16_t* __restrict__ out, const float* __restrict__ S0,
    const float* __restrict__ S1) {
  constexpr int NT = C::NT, STAGES = C::STAGES, BM = C::BM;
  constexpr int GPT = (kMaxGroups + NT - 1) / NT;
  constexpr int OUTC = PHASE == 1 ? C::BN / 2 : C::BN;
  // dynamic LDS: the operand ring, each wave's epilogue block, then per group
  // its first m-tile (fu) and its first row (gl), G + 1 entries each, so
  // finding a tile needs no global load once DMAs are in flight (the compiler
  // would wait for all of them before using such a load)
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
  uint8_t* smem = dyn_lds;
  uint8_t* wst = dyn_lds + C::RING + (threadIdx.x >> 6) * kEpiBytes;   // this wave's epilogue block
  int* fu = reinterpret_cast<int*>(dyn_lds + C::RING + C::NW * kEpiBytes);
  int* gl = fu + plan.G + 1;
  // C::F8: two 1 KiB scale buffers (tile parity) after the ring and the epilogue blocks
  __shared__ __attribute__((aligned(16))) float scl[C::F8 ? 2 * 256 : 1];
  __shared__ int wsum[NT / kWave];
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  if (tid == 0 && blockIdx.x == 0 && plan.diag) *plan.diag = 0;

  // m-tiles per group, exclusive scan -> fu
  {
    int cnt[GPT], ov[GPT][2];
    int sum = 0;
#pragma unroll
    for (int q = 0; q < GPT; ++q) {                    // unconditional loads, all in flight at once
      const int gc = min(tid * GPT + q, plan.G - 1);
      ov[q][0] = plan.offs[gc];
      ov[q][1] = plan.offs[gc + 1];
    }
#pragma unroll
    for (int q = 0; q < GPT; ++q) {
      const int g = tid * GPT + q;
      cnt[q] = 0;
      if (g < plan.G) {
        const int lo = min(max(ov[q][0], 0), plan.n_rows), hi = min(max(ov[q][1], 0), plan.n_rows);
        cnt[q] = (max(0, hi - lo) + BM - 1) / BM;
        gl[g] = lo;
        if (g == plan.G - 1) gl[plan.G] = max(lo, hi);
      }
      sum += cnt[q];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) wsum[w] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int i = 0; i < w; ++i) run += wsum[i];
#pragma unroll
    for (int q = 0; q < GPT; ++q) {
      const int g = tid * GPT + q;
      if (g < plan.G) fu[g] = run;
      run += cnt[q];
    }
    if (tid == NT - 1) fu[plan.G] = run;
    __syncthreads();
  }
  const int nch = (Ncols + OUTC - 1) / OUTC;
  const int items = fu[plan.G] * nch;
  const int per_xcd = static_cast<int>(gridDim.x) / kXcds;
  const int share = (items + kXcds - 1) / kXcds;
  const int x = blockIdx.x % kXcds, slot0 = blockIdx.x / kXcds;
  const int base = x * share;
  // This XCD's L items run in rounds of per_xcd: my full items are
  // base + slot0 + r * per_xcd for r < F.  A last, partly filled round would
  // leave most blocks idle while a few finish a whole tile, so its rem items
  // are cut into `pieces` row ranges of BM / pieces rows (whole 32-row slabs,
  // at most one piece per block) and slot0 takes piece slot0 of that list.
  const int L = max(0, min(share, items - base));
  const int F = L / per_xcd, rem = L % per_xcd;
  int pieces = 1;
  while (rem > 0 && pieces < BM / 32 && rem * pieces * 2 <= per_xcd) pieces *= 2;
  const int prow = BM / pieces;                        // rows per piece
  auto item_of = [&](int want) -> Item {
    const int u = want / nch;                          // global m-tile index
    int lo = 0, hi = plan.G;                           // last g with fu[g] <= u
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (fu[mid] <= u) lo = mid; else hi = mid;
    }
    const int g = lo;
    const int nt = fu[g + 1] - fu[g];
    const int local = want - fu[g] * nch;
    const int j = local / nt, mt = local % nt;
    const int glo = gl[g], ghi = max(glo, gl[g + 1]);
    return contiguous_item(glo + mt * BM, min(BM, ghi - glo - mt * BM), expert_of_group(g, plan.E, plan.nseg), j);
  };
  Item last_piece{};
  bool has_piece = false;
  if (slot0 < rem * pieces) {
    const Item whole = item_of(base + F * per_xcd + slot0 / pieces);
    const int off = (slot0 % pieces) * prow;
    if (off < whole.rows) {                            // pieces past a partial tile's rows are empty
      last_piece = contiguous_item(whole.row0 + off, min(prow, whole.rows - off), whole.expert, whole.chunk);
      has_piece = true;
    }
  }
  const int n_my = F + (has_piece ? 1 : 0);
  if (n_my == 0) return;
  auto decode = [&](int r) -> Item { return r < F ? item_of(base + slot0 + r * per_xcd) : last_piece; };

  const int nk = K / kGemmBK;
  const int total = n_my * nk;                         // K-steps of all my tiles, in order
  const uint32_t lds0 = lds_address(smem);
  // issue side: next K-step to load is step ikt of my tile ir, into ring slot islot
  TileLoader<PHASE, C, PKB> ld;
  int ir = 0, ikt = 0, islot = 0;
  auto issue_next = [&]() {
    if (ikt == 0) {
      ld.init(A, plan.arows, plan.n_x, K, W0, W1, Ncols, decode(ir), S0, S1);
      // one wave loads the tile's scales; its extra load only makes its later
      // waits stricter, and the barrier after the wait that covers it makes
      // the scales visible to every wave long before the epilogue
      if constexpr (C::F8)
        if (w == 0) ld.issue_scales(lds_address(reinterpret_cast<const uint8_t*>(scl + (ir & 1) * 256)));
    }
    ld.issue(ikt, islot, lds0);
    islot = islot + 1 == STAGES ? 0 : islot + 1;
    if (++ikt == nk) {
      ikt = 0;
      ++ir;
    }
  };
  TileMath<PHASE, C, PKB> mm;
  mm.init();
  Item cur{};
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < total) issue_next();
  // compute side: global step gs (tile cr, step gs - cr * nk) from ring slot cslot
  int gs = 0, cslot = 0;
  for (int cr = 0; cr < n_my; ++cr) {
    cur = decode(cr);
    mm.set_rows(cur.rows);
    mm.zero();
    mm.with_nv([&](auto nvc) {
      for (int ckt = 0; ckt < nk; ++ckt, ++gs) {
        // step gs's loads are done once only the later steps' remain in flight
        // (epilogue stores issued since then only make this wait longer)
        wait_ahead_barrier<C::ADMA + C::BDMA, STAGES - 2>(min(STAGES - 2, total - 1 - gs));
        // every wave is past step gs-1, so its buffer can be refilled
        if (gs + STAGES - 1 < total) issue_next();
        mm.template kstep_n<decltype(nvc)::value>(smem + cslot * C::STAGE);
        cslot = cslot + 1 == STAGES ? 0 : cslot + 1;
      }
    });
    if constexpr (C::F8) mm.apply_scales(scl + (cr & 1) * 256);
    mm.store_staged(cur, Ncols, out, wst);
  }
}

// Grid of the persistent GEMM: BLOCKS_PER_CU per CU, a multiple of the XCDs.
int device_cus();

template <class C>
int gemm_grid() {
  const int b = device_cus() * C::BLOCKS_PER_CU;
  return (b + kXcds - 1) / kXcds * kXcds;
}

// ---- mixed batches: one persistent launch, device-side tile queues --------------
// ExpertPlex page, "Adaptive Persistent Kernels (APK)": one resident kernel
// whose workers take tiles from a device-side queue, the urgent decode tiles
// first, so a decode tile waits at most for the tiles already running and no
// host relaunch sits between the two phases.  Both phases run in one launch of
// persistent blocks (two per CU) on 128 x 256 LDS-tiled GEMM tiles (128-row
// units); the tile order is queue_plan.h's:
//   * sequences are experts (with a priority segment an expert's priority rows
//     followed by its other rows), cut into 128-row units;
//   * block b takes its tiles from queue b mod 8 with one atomic add; queue
//     order puts the priority units' phase 1 first and their phase 2 after a
//     lag of one round of the other phase-1 tiles;
//   * a phase-2 tile of unit u waits until each phase-1 tile of u has raised
//     its flag (one int per (unit, column chunk)).
// (Weight-streaming tiles for the experts of <= 64 rows, the decode kernel's
// tile body, ran beside the GEMM tiles in an earlier form of this kernel: on
// the GPT-OSS-shaped mixed batch the call took 1.82 ms against 1.78 ms with
// GEMM tiles only, and the decode segment finished no sooner.)
// Memory ordering (gfx950 under the LLVM AMDGPU memory model, agent scope).
// A phase-1 tile writes its SwiGLU rows with agent-scope atomic stores
// (global_store ... sc1: written through the XCD's L2, so none of them leaves a
// dirty line there); every wave then waits for its stores to complete
// (s_waitcnt vmcnt(0)), the block barriers, and thread 0 stores the flag with an
// agent-scope atomic store.  These are the machine steps of an agent-scope
// release: the release fence's L2 write-back (buffer_wbl2 sc1) finds nothing to
// write back after write-through stores, and its wait is that vmcnt(0).  A
// phase-2 tile's first wave polls the flags with agent-scope atomic loads
// (global_load ... sc1, never served from a stale L2 line); once all are set it
// executes an agent-scope acquire fence (buffer_inv sc1: the XCD's L2 and the
// CU's L1 drop lines that another XCD may have written) and the block
// barriers before any wave loads the rows.  The rows are thus visible to the
// consumer on any XCD, whatever the hardware's placement of the blocks.  The
// argument is at the instruction level: in the language's model the flag store
// is relaxed, and the release is the write-through plus the completion wait.
// Progress: every queue lists all phase-1 tiles a phase-2 tile of it may need
// before that tile, priority ones at the very front, so each awaited tile has
// been or will be popped by a block that is not waiting (queue_plan.h; checked
// for every queue position by a host program built on the same header).
// Every wait is still bounded: it gives up after kWaitTicks of the 100 MHz
// real-time counter (or kMaxPolls polls), or at once when another wait gave
// up; the block then sets the diagnostic word (the workspace's last 4 bytes)
// and waits no more, so a fault of the protocol costs a bounded delay and a
// flagged result, never a hang.
constexpr int kQueueStride = 32;                 // ints between the queue heads (128 B)
constexpr int kMaxQueues = 8;
constexpr unsigned long long kWaitTicks = 2000000ull;   // 20 ms of the 100 MHz counter
constexpr int kMaxPolls = 1 << 22;
constexpr int kMaxSeq = MOE_MAX_EXPERTS_DEV + 256;      // routed + shared experts
constexpr int kSeqPerThread = (kMaxSeq + kThreads - 1) / kThreads;

struct QueueArgs {
  qplan::Shape shape;
  const int* offs;
  const int* arows;   // phase-1 A row list (nullptr: sorted rows)
  int n_x;
  int* heads;         // [nq * kQueueStride]: one head per queue
  int* flags;         // [units_cap][nch1]: phase-1 tile (unit, chunk) done
  int* error;         // diagnostic word, set when a wait gave up
  unsigned long long* trace;   // optional per-tile records, trace_per_queue per queue
  int trace_per_queue;
  const float* s_gate;         // FP8 codes (QC::C::F8): weight-row scales
  const float* s_up;
  const float* s_down;
};

__device__ __forceinline__ unsigned long long realtime() { return __builtin_amdgcn_s_memrealtime(); }

// Configuration of the persistent queue kernel: 128 x 256 GEMM tiles, two
// blocks per CU, on bf16 weights (GemmSmall's ring; row-major with PK false
// or pre-packed) or on packed FP8 codes (GemmSmallF8).
template <bool PKV, class CV = GemmSmall>
struct QueueGemm {
  using C = CV;
  static constexpr int BPC = C::BLOCKS_PER_CU;
  static constexpr bool PK = PKV;
  static constexpr int RING = C::RING;
};

template <class QC>
__global__ __launch_bounds__(kThreads, QC::BPC) void ffn_queue_bf16(
    const uint16_t* __restrict__ x, int d, const uint16_t* __restrict__ w_gate, const uint16_t* __restrict__ w_up,
    const uint16_t* __restrict__ w_down, int I, QueueArgs q, uint16_t* __restrict__ abuf,
    uint16_t* __restrict__ h) {
  using C = typename QC::C;
  static_assert(C::NT == kThreads, "queue blocks have the GEMM tile's shape");
  constexpr int NV = 5;              // per sequence: units, then this queue's P1, R1, P2, R2 tile counts
  // dynamic LDS: the ring (GEMM operands), then NV prefix arrays of nseq + 1
  // ints
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
  uint8_t* smem = dyn_lds;
  const qplan::Shape& sh = q.shape;
  const int ns = sh.nseq();
  int* fu = reinterpret_cast<int*>(dyn_lds + QC::RING);
  __shared__ int wsum[kWaves][NV];
  __shared__ int s_tile, s_ok;
  __shared__ __attribute__((aligned(16))) float scl[C::F8 ? 256 : 1];   // FP8: the tile's row scales
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  const int qi = static_cast<int>(blockIdx.x) % sh.nq;   // block b takes its tiles from queue b mod nq

  {
    int cnt[kSeqPerThread][NV];
    int sum[NV];
#pragma unroll
    for (int c = 0; c < NV; ++c) sum[c] = 0;
#pragma unroll
    for (int i = 0; i < kSeqPerThread; ++i) {
      const int s = tid * kSeqPerThread + i;
#pragma unroll
      for (int c = 0; c < NV; ++c) cnt[i][c] = 0;
      if (s < ns) {
        const qplan::SeqUnits u = qplan::seq_units(sh, qplan::seq_rows(sh, q.offs, s));
        const qplan::SeqCounts c = qplan::seq_counts(sh, s, u, qi);
        cnt[i][0] = u.units;
        cnt[i][1] = c.p1;
        cnt[i][2] = c.r1;
        cnt[i][3] = c.p2;
        cnt[i][4] = c.r2;
      }
#pragma unroll
      for (int c = 0; c < NV; ++c) sum[c] += cnt[i][c];
    }
    int incl[NV];
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      incl[c] = sum[c];
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(incl[c], o, kWave);
        if (lane >= o) incl[c] += y;
      }
      if (lane == kWave - 1) wsum[w][c] = incl[c];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      int run = incl[c] - sum[c];
      for (int i = 0; i < w; ++i) run += wsum[i][c];
      int* arr = fu + c * (ns + 1);
#pragma unroll
      for (int i = 0; i < kSeqPerThread; ++i) {
        const int s = tid * kSeqPerThread + i;
        if (s < ns) arr[s] = run;
        run += cnt[i][c];
      }
      if (tid == kThreads - 1) arr[ns] = run;
    }
    __syncthreads();
  }
  const int nch1 = sh.nch1;
  bool waits = true;                 // false once a wait of this block gave up (block-uniform)
  const int* pre = fu + (ns + 1);    // P1, R1, P2, R2 prefixes of queue qi
  const qplan::QueueParts qp = qplan::queue_parts(
      sh, qplan::SeqCounts{pre[ns], pre[(ns + 1) + ns], pre[2 * (ns + 1) + ns], pre[3 * (ns + 1) + ns]});
  const int total = qp.total();
  for (;;) {
    if (tid == 0) s_tile = __hip_atomic_fetch_add(q.heads + qi * kQueueStride, 1, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();                 // also: every wave is done with the previous tile's LDS
    const int t = s_tile;
    __syncthreads();                 // s_tile read by all before thread 0 overwrites it
    if (t >= total) break;
    const qplan::Slot sl = qplan::slot_of(qp, t);
    const int* pr = pre + ((sl.phase == 1 ? 0 : 2) + (sl.prio ? 0 : 1)) * (ns + 1);
    const qplan::Tile tl = qplan::decode_tile(sh, q.offs, pr, fu, qi, sl);
    const Item it{tl.row0, tl.rows, tl.seq, tl.chunk, tl.split, tl.row1};
    const unsigned long long t0 = q.trace ? realtime() : 0ull;
    if (tl.phase == 1) {
      gemm_tile<1, C, true, QC::PK>(x, q.arows, q.n_x, d, w_gate, w_up, I, it, abuf, smem, q.s_gate, q.s_up, scl);
      // publish: every wave's agent-scope row stores have completed, then the flag
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0)
        __hip_atomic_store(q.flags + static_cast<size_t>(tl.unit) * nch1 + tl.chunk, 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if (waits) {
        if (w == 0) {
          // lane c watches the flags of chunks c, c + 64, ...
          const int* f = q.flags + static_cast<size_t>(tl.unit) * nch1;
          const int nf = nch1;
          const unsigned long long start = realtime();
          int ok = 1, polls = 0;
          for (;;) {
            int mine = 1;
            for (int c = lane; c < nf; c += kWave)
              mine &= __hip_atomic_load(f + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
            if (__all(mine)) break;
            ++polls;
            if (((polls & 63) == 0 && __hip_atomic_load(q.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) ||
                polls > kMaxPolls || realtime() - start > kWaitTicks) {
              ok = 0;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
          if (ok) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          } else if (lane == 0) {
            __hip_atomic_store(q.error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          if (lane == 0) s_ok = ok;
        }
        __syncthreads();
        waits = s_ok != 0;
      }
      gemm_tile<2, C, false, QC::PK>(abuf, nullptr, 0, I, w_down, nullptr, d, it, h, smem, q.s_down, nullptr, scl);
    }
    if (q.trace && tid == 0 && t < q.trace_per_queue) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      unsigned long long* r = q.trace + 4 * (static_cast<size_t>(qi) * q.trace_per_queue + t);
      r[0] = t0;
      r[1] = realtime();
      r[2] = (static_cast<unsigned long long>(tl.unit) << 32) | (static_cast<unsigned long long>(tl.chunk) << 8) |
             (static_cast<unsigned long long>(tl.prio) << 1) |
             static_cast<unsigned long long>(tl.phase - 1);
      r[3] = (static_cast<unsigned long long>(qi) << 32) | blockIdx.x;
    }
  }
}

// Clears the queue heads, the phase-1 flags and the diagnostic word (a kernel,
// not a memset, so the call can sit in a captured graph).
__global__ void ffn_queue_reset(int* p, int n, int* diag) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
  if (i == 0) *diag = 0;
}

// ---- fp32 phase kernel (VALU, fp32 accumulation) --------------------------------
// One thread per output column (256 columns per item), all rows of a 16-row
// tile.
template <int PHASE>
__global__ __launch_bounds__(kThreads) void ffn_phase_f32(const float* __restrict__ A, int K,
                                                          const float* __restrict__ W0, const float* __restrict__ W1,
                                                          int Ncols, PlanArgs plan, float* __restrict__ out) {
  constexpr int BM = 16;
  __shared__ float As[BM * 64];
  const Item it = block_find_item(plan, (Ncols + kThreads - 1) / kThreads);
  if (it.rows == 0) return;
  const int rows = it.rows, e = it.expert;
  const int n = it.chunk * kThreads + threadIdx.x;
  const size_t wstride = static_cast<size_t>(Ncols) * K;
  const float* b0 = W0 + static_cast<size_t>(e) * wstride + static_cast<size_t>(n) * K;
  const float* b1 = PHASE == 1 ? W1 + static_cast<size_t>(e) * wstride + static_cast<size_t>(n) * K : nullptr;
  float acc0[BM], acc1[BM];
#pragma unroll
  for (int r = 0; r < BM; ++r) acc0[r] = acc1[r] = 0.f;
  for (int k0 = 0; k0 < K; k0 += 64) {
    for (int idx = threadIdx.x; idx < BM * 64; idx += kThreads) {
      const int r = idx >> 6, kk = k0 + (idx & 63);
      As[idx] = (r < rows && kk < K) ? A[a_row(plan.arows, plan.n_x, it.row(r)) * K + kk] : 0.f;
    }
    __syncthreads();
    if (n < Ncols) {
      const int kn = min(64, K - k0);
      for (int kk = 0; kk < kn; ++kk) {
        const float w0 = b0[k0 + kk];
        const float w1 = PHASE == 1 ? b1[k0 + kk] : 0.f;
#pragma unroll
        for (int r = 0; r < BM; ++r) {
          acc0[r] += As[r * 64 + kk] * w0;
          if (PHASE == 1) acc1[r] += As[r * 64 + kk] * w1;
        }
      }
    }
    __syncthreads();
  }
  if (n >= Ncols) return;
  for (int r = 0; r < rows; ++r) {
    const float v = PHASE == 1 ? acc0[r] / (1.0f + expf(-acc0[r])) * acc1[r] : acc0[r];
    out[static_cast<size_t>(it.row(r)) * Ncols + n] = v;
  }
}

// ---- host side -------------------------------------------------------------------
enum class Path { kDecode, kGemm, kGemmLarge, kQueue, kF32 };

struct Layout {
  Path path;
  bool splitk;   // decode path: the split-K kernel (groups average <= kSplitKMaxAvg rows)
  int BM, max_tiles;
  size_t a_off, q_off, q_ints, total;
};

// The host never sees the real group sizes: pick the kernel from the average.
// Small groups (decode) stream weights through the decode kernel; large groups
// use the LDS-tiled GEMM, whose K steps need d and I to be multiples of 32
// (otherwise the decode kernel, which takes any multiple of 8, runs them).
// LIBMOE_FFN_QUEUE=0 runs priority batches on the two-launch GEMM instead of
// the persistent queue (for comparisons; the results are the same up to the
// order of nothing: both compute every output from the same products).
bool queue_path_requested() {
  const char* v = getenv("LIBMOE_FFN_QUEUE");
  return v == nullptr || v[0] != '0';
}

// Up to this many rows per group on average the decode path runs the split-K
// kernel (measured on DeepSeek-V2-Lite-shaped decode batches: 3.9 rows per
// group 139 -> 133 us, 1.9 rows 112 -> 99 us; at 4.8 rows it is 2 % slower and
// at 7.8 rows 6 % slower than the whole-K kernel).
constexpr int kSplitKMaxAvg = 4;

int pick_mf(int avg) {
  if (avg <= 8) return 1;
  if (avg <= 24) return 2;
  return 4;
}

// Tile order of the persistent queue for a call (queue_plan.h): 128-row GEMM
// units with 128 SwiGLU / 256 output columns per tile, 64-row stream units with
// 64 / 128 columns per tile.
qplan::Shape queue_shape(int n_rows, int E, int n_shared, int nseg, int d, int I, int nq, int lag) {
  qplan::Shape sh;
  sh.E = E;
  sh.S = n_shared;
  sh.nseg = nseg;
  sh.n_rows = n_rows;
  sh.bm = GemmSmall::BM;
  sh.nch1 = (I + GemmSmall::BN / 2 - 1) / (GemmSmall::BN / 2);
  sh.nch2 = (d + GemmSmall::BN - 1) / GemmSmall::BN;
  sh.nq = nq;
  sh.lag = lag;
  return sh;
}

// Units never exceed ceil(n_rows / bm) + one partial unit per sequence.
int queue_units_cap(const qplan::Shape& sh) { return (sh.n_rows + sh.bm - 1) / sh.bm + sh.nseq(); }

Layout layout(int n_rows, int E, int n_shared, int nseg, int d, int I, int bf16) {
  Layout L;
  const int G = nseg * E + n_shared;
  const int avg = G > 0 ? n_rows / G : n_rows;
  L.splitk = false;
  if (!bf16) {
    L.path = Path::kF32;
    L.BM = 16;
  } else if (avg <= 48 || d % kGemmBK != 0 || I % kGemmBK != 0) {
    L.path = Path::kDecode;
    L.BM = 16 * pick_mf(avg);
    L.splitk = static_cast<long long>(n_rows) <= static_cast<long long>(kSplitKMaxAvg) * G;
    // Decode-sized batches keep two launches: the persistent queue with
    // stream tiles only (both phases in one launch, 16/32/64-row units, four
    // or two blocks per CU) was slower on every decode shape measured
    // (OLMoE-shaped FFN 161 -> 194 us, DSv2-Lite T=128 176 -> 215 us): per tile
    // it adds a queue pop, a completion wait before the flag and written-through
    // intermediate rows, against tiles of a few tens of microseconds.
  } else {
    // With a priority segment both phases run in one persistent launch
    // (ffn_queue_bf16: decode-priority tile queues of GEMM tiles); otherwise
    // two GEMM launches.
    L.path = (nseg > 1 && queue_path_requested()) ? Path::kQueue
             : avg >= kGemmLargeMinAvg                  ? Path::kGemmLarge
                                                        : Path::kGemm;
    L.BM = L.path == Path::kGemmLarge ? GemmLarge::BM : GemmSmall::BM;
  }
  L.max_tiles = (n_rows + L.BM - 1) / L.BM + G;
  L.a_off = 0;
  const size_t a_bytes = static_cast<size_t>(n_rows) * I * (bf16 ? 2 : 4);
  L.q_off = (a_bytes + 255) / 256 * 256;
  // persistent queue: the queue heads, then one phase-1 flag per (unit,
  // column chunk); the last 4 bytes of the workspace are the diagnostic word
  L.q_ints = 0;
  if (L.path == Path::kQueue) {
    const qplan::Shape sh = queue_shape(n_rows, E, n_shared, nseg, d, I, kMaxQueues, 0);
    L.q_ints = static_cast<size_t>(kMaxQueues) * kQueueStride + static_cast<size_t>(queue_units_cap(sh)) * sh.nch1;
  }
  L.total = L.q_off + (L.q_ints * 4 + 255) / 256 * 256 + 256;
  return L;
}

// Decode-kernel shape: 16-column blocks per wave in each phase (the down
// projection gives each wave two blocks so both phases stream two weight rows
// per lane).
constexpr int kDecodeNfc1 = 1;
constexpr int kDecodeNfc2 = 2;

// Groups of at most kSplitKMaxAvg rows on average: the split-K kernel, 16
// columns per item in phase 1 and 32 in phase 2 (tiles of 16 rows).
// Phase-1 plan and combine arguments of a call: with the fused combine
// (a.y32 set) the phase-1 blocks clear the combine sums and the down
// projection adds into them.
PlanArgs phase1_plan(const FfnArgs& a, const PlanArgs& plan) {
  PlanArgs p = plan;
  if (a.y32) {
    p.zero = a.y32;
    p.zero_n4 = static_cast<int>(static_cast<long long>(a.T) * a.d / 4);
  }
  return p;
}

CombineArgs combine_args(const FfnArgs& a) { return CombineArgs{a.s2f, a.topk_w, a.T, a.k, a.n_rows, a.y32}; }

template <bool PK>
void launch_decode_splitk_bf16(const FfnArgs& a, const Layout& L, const PlanArgs& plan, uint16_t* abuf,
                               hipStream_t stream) {
  constexpr int NFC1 = 1, NFC2 = 2;
  const int nch1 = (a.I + 16 * NFC1 - 1) / (16 * NFC1), nch2 = (a.d + 16 * NFC2 - 1) / (16 * NFC2);
  const CombineArgs cmb = combine_args(a);
  hipLaunchKernelGGL((ffn_decode_splitk_bf16<NFC1, 1, PK>), dim3(item_grid(L.max_tiles, nch1)), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(a.x_sorted), a.d, static_cast<const uint16_t*>(a.w_gate),
                     static_cast<const uint16_t*>(a.w_up), a.I, phase1_plan(a, plan), abuf, cmb);
  PlanArgs plan2 = plan;
  plan2.diag = nullptr;
  plan2.arows = nullptr;
  if (a.y32)
    hipLaunchKernelGGL((ffn_decode_splitk_bf16<NFC2, 2, PK, true>), dim3(item_grid(L.max_tiles, nch2)),
                       dim3(kThreads), 0, stream, static_cast<const uint16_t*>(abuf), a.I,
                       static_cast<const uint16_t*>(a.w_down), static_cast<const uint16_t*>(nullptr), a.d, plan2,
                       static_cast<uint16_t*>(nullptr), cmb);
  else
    hipLaunchKernelGGL((ffn_decode_splitk_bf16<NFC2, 2, PK>), dim3(item_grid(L.max_tiles, nch2)), dim3(kThreads), 0,
                       stream, static_cast<const uint16_t*>(abuf), a.I, static_cast<const uint16_t*>(a.w_down),
                       static_cast<const uint16_t*>(nullptr), a.d, plan2, static_cast<uint16_t*>(a.h_sorted), cmb);
}

template <int MF, bool PK>
void launch_decode_bf16(const FfnArgs& a, const Layout& L, const PlanArgs& plan, uint16_t* abuf,
                        hipStream_t stream) {
  const int bn1 = kWaves * 16 * kDecodeNfc1, bn2 = kWaves * 16 * kDecodeNfc2;
  const int nch1 = (a.I + bn1 - 1) / bn1, nch2 = (a.d + bn2 - 1) / bn2;
  const CombineArgs cmb = combine_args(a);
  hipLaunchKernelGGL((ffn_decode_bf16<MF, kDecodeNfc1, 1, PK>), dim3(item_grid(L.max_tiles, nch1)), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(a.x_sorted), a.d, static_cast<const uint16_t*>(a.w_gate),
                     static_cast<const uint16_t*>(a.w_up), a.I, phase1_plan(a, plan), abuf, cmb);
  PlanArgs plan2 = plan;
  plan2.diag = nullptr;
  plan2.arows = nullptr;
  if (a.y32)
    hipLaunchKernelGGL((ffn_decode_bf16<MF, kDecodeNfc2, 2, PK, true>), dim3(item_grid(L.max_tiles, nch2)),
                       dim3(kThreads), 0, stream, static_cast<const uint16_t*>(abuf), a.I,
                       static_cast<const uint16_t*>(a.w_down), static_cast<const uint16_t*>(nullptr), a.d, plan2,
                       static_cast<uint16_t*>(nullptr), cmb);
  else
    hipLaunchKernelGGL((ffn_decode_bf16<MF, kDecodeNfc2, 2, PK>), dim3(item_grid(L.max_tiles, nch2)), dim3(kThreads),
                       0, stream, static_cast<const uint16_t*>(abuf), a.I, static_cast<const uint16_t*>(a.w_down),
                       static_cast<const uint16_t*>(nullptr), a.d, plan2, static_cast<uint16_t*>(a.h_sorted), cmb);
}

template <class C, bool PKB>
void launch_gemm_bf16(const FfnArgs& a, const Layout& L, const PlanArgs& plan, uint16_t* abuf, hipStream_t stream) {
  constexpr int BN = C::BN;
  const int nch1 = (a.I + BN / 2 - 1) / (BN / 2), nch2 = (a.d + BN - 1) / BN;
  PlanArgs plan2 = plan;
  plan2.diag = nullptr;
  plan2.arows = nullptr;
  const uint16_t* x = static_cast<const uint16_t*>(a.x_sorted);
  const uint16_t* wg = static_cast<const uint16_t*>(a.w_gate);
  const uint16_t* wu = static_cast<const uint16_t*>(a.w_up);
  const uint16_t* wd = static_cast<const uint16_t*>(a.w_down);
  uint16_t* h = static_cast<uint16_t*>(a.h_sorted);
  if constexpr (C::BLOCKS_PER_CU > 1) {
    hipLaunchKernelGGL((ffn_gemm_bf16<1, C, PKB>), dim3(item_grid(L.max_tiles, nch1)), dim3(C::NT), 0, stream, x, a.d, wg,
                       wu, a.I, plan, abuf, static_cast<const float*>(nullptr), static_cast<const float*>(nullptr));
    hipLaunchKernelGGL((ffn_gemm_bf16<2, C, PKB>), dim3(item_grid(L.max_tiles, nch2)), dim3(C::NT), 0, stream, abuf, a.I,
                       wd, static_cast<const uint16_t*>(nullptr), a.d, plan2, h, static_cast<const float*>(nullptr),
                       static_cast<const float*>(nullptr));
  } else {
    const size_t lds = C::RING + C::NW * kEpiBytes + 8 * static_cast<size_t>(plan.G + 1);
    hipLaunchKernelGGL((ffn_gemm_persistent_bf16<1, C, PKB>), dim3(gemm_grid<C>()), dim3(C::NT), lds, stream, x, a.d, wg,
                       wu, a.I, plan, abuf, static_cast<const float*>(nullptr), static_cast<const float*>(nullptr));
    hipLaunchKernelGGL((ffn_gemm_persistent_bf16<2, C, PKB>), dim3(gemm_grid<C>()), dim3(C::NT), lds, stream, abuf, a.I,
                       wd, static_cast<const uint16_t*>(nullptr), a.d, plan2, h, static_cast<const float*>(nullptr),
                       static_cast<const float*>(nullptr));
  }
}

// CUs of the current device (cached per device).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  const int slot = dev < 64 ? dev : 63;
  if (cached[slot] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[slot] = cus;
  }
  return cached[slot];
}

template <class QC>
void launch_queue_bf16(const FfnArgs& a, const Layout& L, char* ws, hipStream_t stream) {
  int* qbase = reinterpret_cast<int*>(ws + L.q_off);
  const int n = static_cast<int>(L.q_ints);
  int* diag = reinterpret_cast<int*>(ws + L.total - 4);
  hipLaunchKernelGGL(ffn_queue_reset, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, stream, qbase, n,
                     diag);
  const int blocks = device_cus() * QC::BPC;              // persistent: QC::BPC blocks per CU
  const int nq = blocks >= kMaxQueues ? kMaxQueues : blocks;
  QueueArgs q;
  q.shape = queue_shape(a.n_rows, a.E, a.n_shared, a.nseg, a.d, a.I, nq, (blocks + nq - 1) / nq);
  q.offs = a.group_offsets;
  q.arows = a.x_rows;
  q.n_x = a.n_x;
  q.heads = qbase;
  q.flags = qbase + kMaxQueues * kQueueStride;
  q.error = diag;
  q.trace = a.trace;
  q.trace_per_queue = a.trace ? a.trace_capacity / q.shape.nq : 0;
  q.s_gate = a.s_gate;
  q.s_up = a.s_up;
  q.s_down = a.s_down;
  const size_t lds = QC::RING + 5 * static_cast<size_t>(q.shape.nseq() + 1) * sizeof(int);
  hipLaunchKernelGGL((ffn_queue_bf16<QC>), dim3(blocks), dim3(kThreads), lds, stream,
                     static_cast<const uint16_t*>(a.x_sorted), a.d, static_cast<const uint16_t*>(a.w_gate),
                     static_cast<const uint16_t*>(a.w_up), static_cast<const uint16_t*>(a.w_down), a.I, q,
                     reinterpret_cast<uint16_t*>(ws + L.a_off), static_cast<uint16_t*>(a.h_sorted));
}

// FP8-weight FFN: both phases on the FP8 decode kernel (groups of any size;
// it is the decode-shaped kernel, meant for decode-sized groups).
template <int MF, bool PK>
void launch_decode_fp8w(const FfnArgs& a, int max_tiles, const PlanArgs& plan, uint16_t* abuf,
                        hipStream_t stream) {
  const int bn1 = kWaves8 * 16 * 1, bn2 = kWaves8 * 16 * 2;
  const int nch1 = (a.I + bn1 - 1) / bn1, nch2 = (a.d + bn2 - 1) / bn2;
  hipLaunchKernelGGL((ffn_decode_fp8w<MF, 1, 1, PK>), dim3(item_grid(max_tiles, nch1)), dim3(kThreads8), 0, stream,
                     static_cast<const uint16_t*>(a.x_sorted), a.d, static_cast<const uint8_t*>(a.w_gate),
                     static_cast<const uint8_t*>(a.w_up), a.s_gate, a.s_up, a.I, plan, abuf);
  PlanArgs plan2 = plan;
  plan2.diag = nullptr;
  plan2.arows = nullptr;
  hipLaunchKernelGGL((ffn_decode_fp8w<MF, 2, 2, PK>), dim3(item_grid(max_tiles, nch2)), dim3(kThreads8), 0, stream,
                     static_cast<const uint16_t*>(abuf), a.I, static_cast<const uint8_t*>(a.w_down),
                     static_cast<const uint8_t*>(nullptr), a.s_down, static_cast<const float*>(nullptr), a.d, plan2,
                     static_cast<uint16_t*>(a.h_sorted));
}

}  // namespace

// FP8 workspace: the SwiGLU intermediate [n_rows][I] bf16, then (batches the
// persistent queue may take) the queue heads and phase-1 flags, then the
// diagnostic word at the end.  The layout depends on the shapes only; whether
// the queue runs also needs 16-byte aligned scales (fp8w_uses_gemm).
bool fp8w_queue_shape(int n_rows, int E, int n_shared, int nseg, int d, int I, bool packed) {
  const int G = nseg * E + n_shared;
  return nseg > 1 && queue_path_requested() &&
         fp8w_uses_gemm(n_rows, G, d, I, packed, nullptr, nullptr, nullptr) &&
         (G > 0 ? n_rows / G : n_rows) < kGemmLargeMinAvg;
}

Layout fp8w_layout(int n_rows, int E, int n_shared, int nseg, int d, int I, bool packed) {
  Layout L{};
  L.path = fp8w_queue_shape(n_rows, E, n_shared, nseg, d, I, packed) ? Path::kQueue : Path::kDecode;
  L.a_off = 0;
  L.q_off = (static_cast<size_t>(n_rows) * I * 2 + 255) / 256 * 256;
  L.q_ints = 0;
  if (L.path == Path::kQueue) {
    const qplan::Shape sh = queue_shape(n_rows, E, n_shared, nseg, d, I, kMaxQueues, 0);
    L.q_ints = static_cast<size_t>(kMaxQueues) * kQueueStride + static_cast<size_t>(queue_units_cap(sh)) * sh.nch1;
  }
  L.total = L.q_off + (L.q_ints * 4 + 255) / 256 * 256 + 256;
  return L;
}

size_t ffn_fp8w_workspace_bytes(int n_rows, int E, int n_shared, int nseg, int d, int I, bool packed) {
  return fp8w_layout(n_rows, E, n_shared, nseg, d, I, packed).total;
}

// FP8 codes on the 256 x 256 persistent GEMM (both phases), for batches whose
// groups average more than kFp8GemmMinAvg rows and whose codes are packed.
constexpr int kFp8GemmMinAvg = 48;

// Groups averaging kGemmLargeMinAvg rows or more: the persistent 256 x 256
// kernel; smaller ones: one 128 x 256 tile per block, two blocks per CU.
void launch_gemm_fp8w(const FfnArgs& a, const PlanArgs& plan0, uint16_t* abuf, hipStream_t stream) {
  const int avg = plan0.G > 0 ? a.n_rows / plan0.G : a.n_rows;
  const bool large = avg >= kGemmLargeMinAvg;
  const int BM = large ? GemmLargeF8::BM : GemmSmallF8::BM;
  PlanArgs plan = plan0;
  plan.BM = BM;
  plan.max_tiles = (a.n_rows + BM - 1) / BM + plan.G;
  PlanArgs plan2 = plan;
  plan2.diag = nullptr;
  plan2.arows = nullptr;
  // the kernels read the codes through their weight pointers as bytes
  const uint16_t* x = static_cast<const uint16_t*>(a.x_sorted);
  const uint16_t* wg = static_cast<const uint16_t*>(a.w_gate);
  const uint16_t* wu = static_cast<const uint16_t*>(a.w_up);
  const uint16_t* wd = static_cast<const uint16_t*>(a.w_down);
  uint16_t* h = static_cast<uint16_t*>(a.h_sorted);
  if (large) {
    using C = GemmLargeF8;
    const size_t lds = C::RING + C::NW * kEpiBytes + 8 * static_cast<size_t>(plan.G + 1);
    hipLaunchKernelGGL((ffn_gemm_persistent_bf16<1, C, false>), dim3(gemm_grid<C>()), dim3(C::NT), lds, stream, x,
                       a.d, wg, wu, a.I, plan, abuf, a.s_gate, a.s_up);
    hipLaunchKernelGGL((ffn_gemm_persistent_bf16<2, C, false>), dim3(gemm_grid<C>()), dim3(C::NT), lds, stream, abuf,
                       a.I, wd, static_cast<const uint16_t*>(nullptr), a.d, plan2, h, a.s_down,
                       static_cast<const float*>(nullptr));
  } else {
    using C = GemmSmallF8;
    const int nch1 = (a.I + C::BN / 2 - 1) / (C::BN / 2), nch2 = (a.d + C::BN - 1) / C::BN;
    hipLaunchKernelGGL((ffn_gemm_bf16<1, C, false>), dim3(item_grid(plan.max_tiles, nch1)), dim3(C::NT), 0, stream, x,
                       a.d, wg, wu, a.I, plan, abuf, a.s_gate, a.s_up);
    hipLaunchKernelGGL((ffn_gemm_bf16<2, C, false>), dim3(item_grid(plan.max_tiles, nch2)), dim3(C::NT), 0, stream,
                       abuf, a.I, wd, static_cast<const uint16_t*>(nullptr), a.d, plan2, h, a.s_down,
                       static_cast<const float*>(nullptr));
  }
}

// Needs K >= 128 in both phases (at least four K-steps per tile: a tile's
// scale buffer is refilled only after the tile after it has started) and
// 16-byte aligned scales (they are copied to LDS in 16-byte pieces).
bool fp8w_uses_gemm(int n_rows, int G, int d, int I, bool packed, const void* s_gate, const void* s_up,
                    const void* s_down) {
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  return packed && d % 64 == 0 && I % 64 == 0 && d >= 128 && I >= 128 && al16(s_gate) && al16(s_up) &&
         al16(s_down) && (G > 0 ? n_rows / G : n_rows) > kFp8GemmMinAvg;
}

hipError_t launch_ffn_fp8w(const FfnArgs& a, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  const Layout L = fp8w_layout(a.n_rows, a.E, a.n_shared, a.nseg, a.d, a.I, a.packed);
  const size_t total = L.total;
  const int G = a.nseg * a.E + a.n_shared;
  const int mf = pick_mf(G > 0 ? a.n_rows / G : a.n_rows);
  PlanArgs plan;
  plan.offs = a.group_offsets;
  plan.G = G;
  plan.E = a.E;
  plan.nseg = a.nseg;
  plan.BM = 16 * mf;
  plan.n_rows = a.n_rows;
  plan.max_tiles = (a.n_rows + plan.BM - 1) / plan.BM + G;
  plan.diag = reinterpret_cast<int*>(ws + total - 4);
  plan.arows = a.x_rows;
  plan.n_x = a.n_x;
  uint16_t* abuf = reinterpret_cast<uint16_t*>(ws);
  if (fp8w_uses_gemm(a.n_rows, G, a.d, a.I, a.packed, a.s_gate, a.s_up, a.s_down)) {
    // a priority segment: both phases in the persistent queue (decode tiles first)
    if (L.path == Path::kQueue) launch_queue_bf16<QueueGemm<false, GemmSmallF8>>(a, L, ws, stream);
    else launch_gemm_fp8w(a, plan, abuf, stream);
    return hipGetLastError();
  }
  if (a.packed) {
    switch (mf) {
      case 1: launch_decode_fp8w<1, true>(a, plan.max_tiles, plan, abuf, stream); break;
      case 2: launch_decode_fp8w<2, true>(a, plan.max_tiles, plan, abuf, stream); break;
      default: launch_decode_fp8w<4, true>(a, plan.max_tiles, plan, abuf, stream); break;
    }
    return hipGetLastError();
  }
  switch (mf) {
    case 1: launch_decode_fp8w<1, false>(a, plan.max_tiles, plan, abuf, stream); break;
    case 2: launch_decode_fp8w<2, false>(a, plan.max_tiles, plan, abuf, stream); break;
    default: launch_decode_fp8w<4, false>(a, plan.max_tiles, plan, abuf, stream); break;
  }
  return hipGetLastError();
}

size_t ffn_workspace_bytes(int n_rows, int E, int n_shared, int nseg, int d, int I, int bf16) {
  return layout(n_rows, E, n_shared, nseg, d, I, bf16).total;
}

hipError_t launch_ffn(const FfnArgs& a, void* workspace, hipStream_t stream) {
  const Layout L = layout(a.n_rows, a.E, a.n_shared, a.nseg, a.d, a.I, a.bf16);
  char* ws = static_cast<char*>(workspace);
  PlanArgs plan;
  plan.offs = a.group_offsets;
  plan.G = a.nseg * a.E + a.n_shared;
  plan.E = a.E;
  plan.nseg = a.nseg;
  plan.BM = L.BM;
  plan.n_rows = a.n_rows;
  plan.max_tiles = L.max_tiles;
  plan.diag = reinterpret_cast<int*>(ws + L.total - 4);
  plan.arows = a.x_rows;
  plan.n_x = a.n_x;
  if (a.packed && L.path == Path::kF32) return hipErrorInvalidValue;
  if (a.y32 && L.path != Path::kDecode) return hipErrorInvalidValue;
  switch (L.path) {
    case Path::kDecode: {
      uint16_t* abuf = reinterpret_cast<uint16_t*>(ws + L.a_off);
      if (a.packed) {
        switch (L.BM / 16) {
          case 1:
            if (L.splitk) launch_decode_splitk_bf16<true>(a, L, plan, abuf, stream);
            else launch_decode_bf16<1, true>(a, L, plan, abuf, stream);
            break;
          case 2: launch_decode_bf16<2, true>(a, L, plan, abuf, stream); break;
          default: launch_decode_bf16<4, true>(a, L, plan, abuf, stream); break;
        }
        break;
      }
      switch (L.BM / 16) {
        case 1:
          if (L.splitk) launch_decode_splitk_bf16<false>(a, L, plan, abuf, stream);
          else launch_decode_bf16<1, false>(a, L, plan, abuf, stream);
          break;
        case 2: launch_decode_bf16<2, false>(a, L, plan, abuf, stream); break;
        default: launch_decode_bf16<4, false>(a, L, plan, abuf, stream); break;
      }
      break;
    }
    case Path::kGemm:
      if (a.packed) launch_gemm_bf16<GemmSmall, true>(a, L, plan, reinterpret_cast<uint16_t*>(ws + L.a_off), stream);
      else launch_gemm_bf16<GemmSmall, false>(a, L, plan, reinterpret_cast<uint16_t*>(ws + L.a_off), stream);
      break;
    case Path::kGemmLarge:
      if (a.packed) launch_gemm_bf16<GemmLarge, true>(a, L, plan, reinterpret_cast<uint16_t*>(ws + L.a_off), stream);
      else launch_gemm_bf16<GemmLarge, false>(a, L, plan, reinterpret_cast<uint16_t*>(ws + L.a_off), stream);
      break;
    case Path::kQueue:
      if (a.packed) launch_queue_bf16<QueueGemm<true>>(a, L, ws, stream);
      else launch_queue_bf16<QueueGemm<false>>(a, L, ws, stream);
      break;
    case Path::kF32: {
      float* abuf = reinterpret_cast<float*>(ws + L.a_off);
      const int nch1 = (a.I + kThreads - 1) / kThreads, nch2 = (a.d + kThreads - 1) / kThreads;
      hipLaunchKernelGGL(ffn_phase_f32<1>, dim3(item_grid(L.max_tiles, nch1)), dim3(kThreads), 0, stream,
                         static_cast<const float*>(a.x_sorted), a.d, static_cast<const float*>(a.w_gate),
                         static_cast<const float*>(a.w_up), a.I, plan, abuf);
      PlanArgs plan2 = plan;
      plan2.diag = nullptr;
      plan2.arows = nullptr;
      hipLaunchKernelGGL(ffn_phase_f32<2>, dim3(item_grid(L.max_tiles, nch2)), dim3(kThreads), 0, stream,
                         static_cast<const float*>(abuf), a.I, static_cast<const float*>(a.w_down),
                         static_cast<const float*>(nullptr), a.d, plan2, static_cast<float*>(a.h_sorted));
      break;
    }
  }
  if (a.y32) {
    const int n8 = static_cast<int>(static_cast<long long>(a.T) * a.d / 8);
    hipLaunchKernelGGL(ffn_combine_finalize, dim3((n8 + kThreads - 1) / kThreads), dim3(kThreads), 0, stream, a.y32,
                       static_cast<uint16_t*>(a.y), n8);
  }
  return hipGetLastError();
}

bool ffn_fused_combine_supported(int n_rows, int E, int n_shared, int nseg, int d, int I) {
  return layout(n_rows, E, n_shared, nseg, d, I, 1).path == Path::kDecode;
}

}  // namespace moe
