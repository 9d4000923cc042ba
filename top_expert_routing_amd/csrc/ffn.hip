// Grouped SwiGLU expert FFN on bf16 MFMA (gfx950), plus an fp32 path.
//
// ExpertPlex page, "Instance vs module disaggregation": the expert FFN is the
// bulk of a MoE layer; ELDR page, "What it solves": a decode step must read the
// weights of every distinct expert the batch selected - and only those.
//
// Work is cut into tiles (group, block of rows, block of output columns).  The
// tile list is built on the device from group_offsets (empty groups give no
// tiles, so unused experts' weights are never read), then two launches run
// the phases:
//   phase 1  a[n][i] = silu(xs[n] . W_gate[e][i]) * (xs[n] . W_up[e][i])  -> bf16
//   phase 2  h[n][o] = a[n] . W_down[e][o]
// Both are C = A B^T with A and B contiguous along K, which is exactly the
// operand layout of v_mfma_f32_16x16x32_bf16: each lane holds 8 consecutive K
// values of one row of A and of one row of B.  The token rows (A) of a tile
// are staged in LDS and shared by the four waves; the weight rows (B) are
// used by exactly one wave, so they stream straight from HBM into registers
// with 16-byte loads and no LDS round trip.
#include "common.h"
#include "launch.h"

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
// Items are ordered group-major: for each group g, for each column chunk j,
// for each m-tile of g - so consecutive items share a group's weight slab (and,
// for one m-tile, its token rows).  Workgroups are dealt round-robin to the
// 8 XCDs (blockIdx % 8), and XCD x takes the x-th eighth of the item list in
// order, so a group's items run close together in one XCD's L2.  The list is
// in group order, so the priority segment's items start first on every XCD
// that holds some.
constexpr int kMaxGroupsPerThread = 5;   // 256 * 5 >= 2*512 + 256 shared groups
constexpr int kXcds = 8;                 // MI355X: 8 XCDs, workgroups dealt round-robin

struct PlanArgs {
  const int* offs;
  int G, E, nseg, BM, n_rows, max_tiles;
};

struct Item {
  int row0, rows, expert, chunk;   // rows == 0: no work for this block
};

// Must be called by all threads of a 256-thread block.
__device__ Item block_find_item(const PlanArgs& p, int nch) {
  __shared__ int wsum[kThreads / kWave];
  __shared__ Item found;
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  if (tid == 0) found = Item{0, 0, 0, 0};
  int cnt[kMaxGroupsPerThread], r0[kMaxGroupsPerThread];
  int s = 0;
#pragma unroll
  for (int q = 0; q < kMaxGroupsPerThread; ++q) {
    const int g = tid * kMaxGroupsPerThread + q;
    cnt[q] = 0;
    r0[q] = 0;
    if (g < p.G) {
      const int lo = min(max(p.offs[g], 0), p.n_rows);
      const int hi = min(max(p.offs[g + 1], 0), p.n_rows);
      r0[q] = lo;
      cnt[q] = max(0, hi - lo);
    }
    s += (cnt[q] + p.BM - 1) / p.BM;
  }
  int incl = s;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) wsum[w] = incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i) {
    base += i < w ? wsum[i] : 0;
    total += wsum[i];
  }
  // this block's item: the x-th eighth of the list, slot s within it
  const long long items = static_cast<long long>(total) * nch;
  const long long share = (items + kXcds - 1) / kXcds;
  const long long slot = blockIdx.x / kXcds;
  const long long want = (blockIdx.x % kXcds) * share + slot;
  if (slot < share && want < items) {
    int t = base + incl - s;     // first m-tile of this thread's first group
#pragma unroll
    for (int q = 0; q < kMaxGroupsPerThread; ++q) {
      const int g = tid * kMaxGroupsPerThread + q;
      if (g >= p.G) break;
      const int nt = (cnt[q] + p.BM - 1) / p.BM;
      const long long first = static_cast<long long>(t) * nch;
      if (nt > 0 && want >= first && want < first + static_cast<long long>(nt) * nch) {
        const int local = static_cast<int>(want - first);
        const int j = local / nt, m = (local % nt) * p.BM;
        found = Item{r0[q] + m, min(p.BM, cnt[q] - m), expert_of_group(g, p.E, p.nseg), j};
      }
      t += nt;
    }
  }
  __syncthreads();
  return found;
}

// Grid size that covers every possible item of a call.
inline int item_grid(int max_tiles, int nch) {
  const long long items = static_cast<long long>(max_tiles) * nch;
  return static_cast<int>((items + kXcds - 1) / kXcds * kXcds);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Weight row of local row `lr` of a weight tile whose output columns start at
// `n0`: phase 1 tiles hold `half` gate rows then the matching `half` up rows,
// phase 2 tiles hold down rows.  Returns nullptr past the last column.
template <int PHASE>
__device__ __forceinline__ const uint16_t* weight_row(const uint16_t* W0, const uint16_t* W1, size_t expert_off,
                                                      int Ncols, int K, int n0, int lr, int half) {
  int n = n0 + lr;
  const uint16_t* W = W0;
  if (PHASE == 1 && lr >= half) {
    n -= half;
    W = W1;
  }
  if (n >= Ncols) return nullptr;
  return W + expert_off + static_cast<size_t>(n) * K;
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
constexpr int kDecodeKC = 256;                 // K per chunk (8 MFMA K-steps)
constexpr int kDecodeStride = kDecodeKC + 8;   // bf16 per staged A row (pad 16 B)
constexpr int kDecodeWavesPerSimd = 4;

template <int MF, int NFC, int PHASE>
__global__ __launch_bounds__(kThreads, MF <= 2 ? kDecodeWavesPerSimd : 2) void ffn_decode_bf16(
    const uint16_t* __restrict__ A, int K, const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
    int Ncols, PlanArgs plan, uint16_t* __restrict__ out) {
  constexpr int NF = PHASE == 1 ? 2 * NFC : NFC;
  constexpr int BN = kWaves * 16 * NFC;
  constexpr int BM = 16 * MF;
  constexpr int U = kDecodeKC / 32;
  constexpr int VPR = kDecodeKC / 8;                       // uint4 per staged row
  constexpr int APT = (BM * VPR + kThreads - 1) / kThreads; // uint4 staged per thread
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kDecodeStride];

  const int nch = (Ncols + BN - 1) / BN;
  const Item it = block_find_item(plan, nch);
  if (it.rows == 0) return;
  const int row0 = it.row0, rows = it.rows, e = it.expert;
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
    bp[j] = W + static_cast<size_t>(e) * wstride + static_cast<size_t>(n) * K + 8 * q;
  }

  // A staging: thread handles uint4 slots idx = tid + s*256 of the chunk
  uint4 stage[APT];
  auto load_a = [&](int c) {
#pragma unroll
    for (int s = 0; s < APT; ++s) {
      const int idx = threadIdx.x + s * kThreads;
      const int r = idx / VPR, kv = idx % VPR;
      const int k = c * kDecodeKC + kv * 8;
      stage[s] = make_uint4(0, 0, 0, 0);
      if (idx < BM * VPR && r < rows && k < K)
        stage[s] = *reinterpret_cast<const uint4*>(A + static_cast<size_t>(row0 + r) * K + k);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int s = 0; s < APT; ++s) {
      const int idx = threadIdx.x + s * kThreads;
      if (idx < BM * VPR)
        *reinterpret_cast<uint4*>(&As[buf][(idx / VPR) * kDecodeStride + (idx % VPR) * 8]) = stage[s];
    }
  };

  f32x4 acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_a(0);
  store_a(0);
  for (int c = 0; c < nchunks; ++c) {
    const int kc = c * kDecodeKC;
    uint4 b[U][NF];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = kc + 32 * u + 8 * q;    // a lane's 8 values are all in range or all out
#pragma unroll
      for (int j = 0; j < NF; ++j)
        b[u][j] = kk < K ? *reinterpret_cast<const uint4*>(bp[j] + kc + 32 * u) : make_uint4(0, 0, 0, 0);
    }
    const bool more = c + 1 < nchunks;
    if (more) load_a(c + 1);
    __syncthreads();                           // chunk c of A is in As[c & 1]
    const uint16_t* as = As[c & 1];
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
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], __builtin_bit_cast(bf16x8, b[u][j]), acc[i][j], 0, 0, 0);
    }
    if (more) store_a((c + 1) & 1);            // that buffer was last read before this barrier
  }

  // lane holds column l16 and rows 4q..4q+3 of each 16x16 block
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NFC; ++j) {
      const int n = col0 + j * 16 + l16;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int m = 16 * i + 4 * q + rr;
        if (m < rows && n < Ncols) {
          const float v = PHASE == 1 ? silu_mul(acc[i][j][rr], acc[i][NFC + j][rr]) : acc[i][j][rr];
          out[static_cast<size_t>(row0 + m) * Ncols + n] = f32_to_bf16(v);
        }
      }
    }
}

// ---- prefill-sized tiles: LDS-tiled GEMM on v_mfma_f32_32x32x16_bf16 ------------
// Block tile: 128 token rows x 128 weight rows (phase 1: 64 gate + the matching
// 64 up rows -> 64 SwiGLU columns; phase 2: 128 down rows), K in steps of 64.
// Both tiles go global -> registers -> LDS, double buffered: the next K-step's
// loads are in flight while the current one is multiplied; one barrier per
// step.  Four waves in a 2 x 2 grid, each 64 x 64 (2 x 2 MFMA 32x32 blocks;
// phase 1: 32 gate and the same 32 up columns, so SwiGLU needs no exchange).
constexpr int kGemmBM = 128;
constexpr int kGemmBN = 128;               // weight rows per tile
constexpr int kGemmBK = 64;
constexpr int kGemmStride = kGemmBK + 8;   // bf16 per LDS row (144 B)
constexpr int kGemmVecs = kGemmBM * kGemmBK / 8 / kThreads;   // uint4 per thread per tile (4)

template <int PHASE>
__global__ __launch_bounds__(kThreads, 2) void ffn_gemm_bf16(
    const uint16_t* __restrict__ A, int K, const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
    int Ncols, PlanArgs plan, uint16_t* __restrict__ out) {
  constexpr int OUTC = PHASE == 1 ? kGemmBN / 2 : kGemmBN;   // output columns per tile
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kGemmBM * kGemmStride];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kGemmBN * kGemmStride];

  const int nch = (Ncols + OUTC - 1) / OUTC;
  const Item it = block_find_item(plan, nch);
  if (it.rows == 0) return;
  const int row0 = it.row0, rows = it.rows;
  const int n0 = it.chunk * OUTC;
  const size_t eoff = static_cast<size_t>(it.expert) * Ncols * K;
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hk = lane >> 5;

  // global -> register staging: slot s of thread t covers row (t + 256 s) / 8, 8 bf16 at column 8 * (t % 8)
  const uint16_t* arow[kGemmVecs];
  const uint16_t* brow[kGemmVecs];
#pragma unroll
  for (int s = 0; s < kGemmVecs; ++s) {
    const int r = (tid + s * kThreads) >> 3;
    arow[s] = r < rows ? A + static_cast<size_t>(row0 + r) * K : nullptr;
    brow[s] = weight_row<PHASE>(W0, W1, eoff, Ncols, K, n0, r, OUTC);
  }
  const int kcol = 8 * (tid & 7);
  uint4 ra[kGemmVecs], rb[kGemmVecs];
  auto load = [&](int k0) {
    const int k = k0 + kcol;
#pragma unroll
    for (int s = 0; s < kGemmVecs; ++s) {
      ra[s] = (arow[s] && k < K) ? *reinterpret_cast<const uint4*>(arow[s] + k) : make_uint4(0, 0, 0, 0);
      rb[s] = (brow[s] && k < K) ? *reinterpret_cast<const uint4*>(brow[s] + k) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int s = 0; s < kGemmVecs; ++s) {
      const int r = (tid + s * kThreads) >> 3;
      *reinterpret_cast<uint4*>(&As[buf][r * kGemmStride + kcol]) = ra[s];
      *reinterpret_cast<uint4*>(&Bs[buf][r * kGemmStride + kcol]) = rb[s];
    }
  };

  // MFMA operand rows of this wave: A rows 64 wm + 32 i + l32; B (weight)
  // rows: phase 2 64 wn + 32 j + l32, phase 1 j = 0 gate 32 wn + l32, j = 1
  // the matching up row 64 + 32 wn + l32.
  int brl[2];
  brl[0] = PHASE == 1 ? 32 * wn + l32 : 64 * wn + l32;
  brl[1] = PHASE == 1 ? 64 + 32 * wn + l32 : 64 * wn + 32 + l32;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + kGemmBK - 1) / kGemmBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) load((kt + 1) * kGemmBK);
    const uint16_t* as = As[kt & 1];
    const uint16_t* bs = Bs[kt & 1];
#pragma unroll
    for (int ks = 0; ks < kGemmBK; ks += 16) {
      bf16x8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&as[(64 * wm + 32 * i + l32) * kGemmStride + ks + 8 * hk]));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&bs[brl[j] * kGemmStride + ks + 8 * hk]));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (more) store((kt + 1) & 1);   // that buffer was last read before the previous barrier
    __syncthreads();
  }

  // 32x32 accumulator: lane holds column l32 and rows 8 (r/4) + 4 hk + r % 4
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * hk + (r & 3);
      if (m >= rows) continue;
      uint16_t* orow = out + static_cast<size_t>(row0 + m) * Ncols;
      if (PHASE == 1) {
        const int n = n0 + 32 * wn + l32;
        if (n < Ncols) orow[n] = f32_to_bf16(silu_mul(acc[i][0][r], acc[i][1][r]));
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + 64 * wn + 32 * j + l32;
          if (n < Ncols) orow[n] = f32_to_bf16(acc[i][j][r]);
        }
      }
    }
  }
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
  const int row0 = it.row0, rows = it.rows, e = it.expert;
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
      As[idx] = (r < rows && kk < K) ? A[static_cast<size_t>(row0 + r) * K + kk] : 0.f;
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
    out[static_cast<size_t>(row0 + r) * Ncols + n] = v;
  }
}

// ---- host side -------------------------------------------------------------------
enum class Path { kDecode, kGemm, kF32 };

struct Layout {
  Path path;
  int BM, max_tiles;
  size_t a_off, total;
};

// The host never sees the real group sizes: pick the kernel from the average.
// Small groups (decode) stream weights through the decode kernel; large groups
// use the LDS-tiled GEMM.
int pick_mf(int avg) {
  if (avg <= 8) return 1;
  if (avg <= 24) return 2;
  return 4;
}

Layout layout(int n_rows, int E, int n_shared, int nseg, int d, int I, int bf16) {
  (void)d;
  Layout L;
  const int G = nseg * E + n_shared;
  const int avg = G > 0 ? n_rows / G : n_rows;
  if (!bf16) {
    L.path = Path::kF32;
    L.BM = 16;
  } else if (avg <= 48) {
    L.path = Path::kDecode;
    L.BM = 16 * pick_mf(avg);
  } else {
    L.path = Path::kGemm;
    L.BM = kGemmBM;
  }
  L.max_tiles = (n_rows + L.BM - 1) / L.BM + G;
  L.a_off = 0;
  const size_t a_bytes = static_cast<size_t>(n_rows) * I * (bf16 ? 2 : 4);
  L.total = (a_bytes + 255) / 256 * 256 + 256;
  return L;
}

// Decode-kernel shape: 16-column blocks per wave in each phase (the down
// projection gives each wave two blocks so both phases stream two weight rows
// per lane).
constexpr int kDecodeNfc1 = 1;
constexpr int kDecodeNfc2 = 2;

template <int MF>
void launch_decode_bf16(const FfnArgs& a, const Layout& L, const PlanArgs& plan, uint16_t* abuf,
                        hipStream_t stream) {
  const int bn1 = kWaves * 16 * kDecodeNfc1, bn2 = kWaves * 16 * kDecodeNfc2;
  const int nch1 = (a.I + bn1 - 1) / bn1, nch2 = (a.d + bn2 - 1) / bn2;
  hipLaunchKernelGGL((ffn_decode_bf16<MF, kDecodeNfc1, 1>), dim3(item_grid(L.max_tiles, nch1)), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(a.x_sorted), a.d, static_cast<const uint16_t*>(a.w_gate),
                     static_cast<const uint16_t*>(a.w_up), a.I, plan, abuf);
  hipLaunchKernelGGL((ffn_decode_bf16<MF, kDecodeNfc2, 2>), dim3(item_grid(L.max_tiles, nch2)), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(abuf), a.I, static_cast<const uint16_t*>(a.w_down),
                     static_cast<const uint16_t*>(nullptr), a.d, plan, static_cast<uint16_t*>(a.h_sorted));
}

void launch_gemm_bf16(const FfnArgs& a, const Layout& L, const PlanArgs& plan, uint16_t* abuf, hipStream_t stream) {
  const int nch1 = (a.I + kGemmBN / 2 - 1) / (kGemmBN / 2), nch2 = (a.d + kGemmBN - 1) / kGemmBN;
  hipLaunchKernelGGL(ffn_gemm_bf16<1>, dim3(item_grid(L.max_tiles, nch1)), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(a.x_sorted), a.d, static_cast<const uint16_t*>(a.w_gate),
                     static_cast<const uint16_t*>(a.w_up), a.I, plan, abuf);
  hipLaunchKernelGGL(ffn_gemm_bf16<2>, dim3(item_grid(L.max_tiles, nch2)), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(abuf), a.I, static_cast<const uint16_t*>(a.w_down),
                     static_cast<const uint16_t*>(nullptr), a.d, plan, static_cast<uint16_t*>(a.h_sorted));
}

}  // namespace

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
  switch (L.path) {
    case Path::kDecode: {
      uint16_t* abuf = reinterpret_cast<uint16_t*>(ws + L.a_off);
      switch (L.BM / 16) {
        case 1: launch_decode_bf16<1>(a, L, plan, abuf, stream); break;
        case 2: launch_decode_bf16<2>(a, L, plan, abuf, stream); break;
        default: launch_decode_bf16<4>(a, L, plan, abuf, stream); break;
      }
      break;
    }
    case Path::kGemm:
      launch_gemm_bf16(a, L, plan, reinterpret_cast<uint16_t*>(ws + L.a_off), stream);
      break;
    case Path::kF32: {
      float* abuf = reinterpret_cast<float*>(ws + L.a_off);
      const int nch1 = (a.I + kThreads - 1) / kThreads, nch2 = (a.d + kThreads - 1) / kThreads;
      hipLaunchKernelGGL(ffn_phase_f32<1>, dim3(item_grid(L.max_tiles, nch1)), dim3(kThreads), 0, stream,
                         static_cast<const float*>(a.x_sorted), a.d, static_cast<const float*>(a.w_gate),
                         static_cast<const float*>(a.w_up), a.I, plan, abuf);
      hipLaunchKernelGGL(ffn_phase_f32<2>, dim3(item_grid(L.max_tiles, nch2)), dim3(kThreads), 0, stream,
                         static_cast<const float*>(abuf), a.I, static_cast<const float*>(a.w_down),
                         static_cast<const float*>(nullptr), a.d, plan, static_cast<float*>(a.h_sorted));
      break;
    }
  }
  return hipGetLastError();
}

}  // namespace moe
