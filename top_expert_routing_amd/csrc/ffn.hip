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
constexpr int kKC = 64;               // K elements staged per LDS chunk
constexpr int kLdsStride = kKC + 8;   // bf16 elements per staged row (pad 16 B)

struct Tile {
  int g, row0, rows, expert;
};

// ---- tile list: one entry per (group, block of BM rows) -----------------------
// One 256-thread block: per-group tile counts, a block-wide exclusive scan,
// then the tile descriptors.  group_offsets is a precondition (non-decreasing, last entry
// n_rows); rows are still clamped to [0, n_rows] and the list to max_tiles so
// that a bad input cannot make a tile reach outside the buffers.
constexpr int kPlanThreads = 256;
constexpr int kMaxGroupsPerThread = 5;   // 256 * 5 >= 2*512 + 256 shared groups

__global__ __launch_bounds__(kPlanThreads) void ffn_plan(const int* __restrict__ offs, int G, int E, int nseg,
                                                         int BM, int n_rows, int max_tiles,
                                                         int4* __restrict__ tiles, int* __restrict__ ntiles) {
  __shared__ int wsum[kPlanThreads / kWave];
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
  int cnt[kMaxGroupsPerThread], r0[kMaxGroupsPerThread];
  int s = 0;
#pragma unroll
  for (int q = 0; q < kMaxGroupsPerThread; ++q) {
    const int g = tid * kMaxGroupsPerThread + q;
    cnt[q] = 0;
    r0[q] = 0;
    if (g < G) {
      const int lo = min(max(offs[g], 0), n_rows);
      const int hi = min(max(offs[g + 1], 0), n_rows);
      r0[q] = lo;
      cnt[q] = max(0, hi - lo);
    }
    s += (cnt[q] + BM - 1) / BM;
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
  for (int i = 0; i < kPlanThreads / kWave; ++i) {
    base += i < w ? wsum[i] : 0;
    total += wsum[i];
  }
  int t = base + incl - s;
#pragma unroll
  for (int q = 0; q < kMaxGroupsPerThread; ++q) {
    const int g = tid * kMaxGroupsPerThread + q;
    if (g >= G) break;
    const int e = expert_of_group(g, E, nseg);
    for (int m = 0; m < cnt[q] && t < max_tiles; m += BM) tiles[t++] = make_int4(g, r0[q] + m, min(BM, cnt[q] - m), e);
  }
  if (tid == 0) *ntiles = min(total, max_tiles);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// ---- bf16 MFMA phase kernel ------------------------------------------------------
// MF: 16-row MFMA blocks per tile (BM = 16*MF).  NFC: 16-column blocks per wave
// per weight matrix.  PHASE 1 multiplies by W_gate and W_up (2*NFC column
// blocks per wave) and applies SwiGLU; PHASE 2 multiplies by W_down.
template <int MF, int NFC, int PHASE>
__global__ __launch_bounds__(kThreads) void ffn_phase_bf16(
    const uint16_t* __restrict__ A, int K, const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
    int Ncols, const int4* __restrict__ tiles, const int* __restrict__ ntiles, uint16_t* __restrict__ out) {
  constexpr int NF = PHASE == 1 ? 2 * NFC : NFC;
  constexpr int BM = 16 * MF;
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * kLdsStride];

  const int tile_id = blockIdx.x;
  if (tile_id >= *ntiles) return;
  const int4 td = tiles[tile_id];
  const int row0 = td.y, rows = td.z, e = td.w;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int l16 = lane & 15, q = lane >> 4;
  const int col_base = blockIdx.y * (kWaves * 16 * NFC) + wave * 16 * NFC;

  const size_t wstride = static_cast<size_t>(Ncols) * K;   // elements per expert matrix
  const uint16_t* B0 = W0 + static_cast<size_t>(e) * wstride;
  const uint16_t* B1 = PHASE == 1 ? W1 + static_cast<size_t>(e) * wstride : nullptr;

  f32x4 acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += kKC) {
    // stage A rows [row0, row0+rows) x K [k0, k0+64) into LDS (zero padded)
    for (int idx = threadIdx.x; idx < BM * (kKC / 8); idx += kThreads) {
      const int r = idx >> 3, kv = idx & 7;
      const int kk = k0 + kv * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < rows && kk < K) v = *reinterpret_cast<const uint4*>(A + static_cast<size_t>(row0 + r) * K + kk);
      *reinterpret_cast<uint4*>(&As[r * kLdsStride + kv * 8]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kKC; ks += 32) {
      const int kk = k0 + ks + q * 8;
      bf16x8 bfr[NF];
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const int n = col_base + (j % NFC) * 16 + l16;
        const uint16_t* B = (PHASE == 1 && j >= NFC) ? B1 : B0;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n < Ncols && kk < K) v = *reinterpret_cast<const uint4*>(B + static_cast<size_t>(n) * K + kk);
        bfr[j] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        const uint4 av = *reinterpret_cast<const uint4*>(&As[(i * 16 + l16) * kLdsStride + ks + q * 8]);
        const bf16x8 afr = __builtin_bit_cast(bf16x8, av);
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds column l16 and rows 4q..4q+3 of each 16x16 block
#pragma unroll
  for (int i = 0; i < MF; ++i) {
#pragma unroll
    for (int j = 0; j < NFC; ++j) {
      const int n = col_base + j * 16 + l16;
      if (n >= Ncols) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = i * 16 + q * 4 + r;
        if (m >= rows) continue;
        float v;
        if (PHASE == 1)
          v = silu_mul(acc[i][j][r], acc[i][NFC + j][r]);
        else
          v = acc[i][j][r];
        out[static_cast<size_t>(row0 + m) * Ncols + n] = f32_to_bf16(v);
      }
    }
  }
}

// ---- decode-sized tiles: weights stream from HBM straight into MFMA registers ----
// One block of four waves per (m-tile of <= 16*MF rows, 64*NFC output columns),
// blocks ordered tile-major.  Each wave computes every row of the m-tile
// against its own 16*NFC columns (phase 1: of W_gate and of W_up).
//   * Weight rows (B) are read exactly once per m-tile, straight into the MFMA
//     B operand: a lane loads 16 bytes of one row; the kDecodeKC/32 K-steps of
//     a chunk are issued back to back, so each row streams in runs of
//     kDecodeKC*2 bytes with many loads in flight.  No LDS round trip.
//   * The few token rows (A) are shared by the four waves: staged through LDS
//     one K-chunk at a time, double buffered, loaded from global while the
//     previous chunk is multiplied.  One barrier per chunk.
// Latency is hidden by the chunk-deep weight loads and the other resident
// blocks.
constexpr int kDecodeKC = 256;                 // K per chunk (8 MFMA K-steps)
constexpr int kDecodeStride = kDecodeKC + 8;   // bf16 per staged A row (pad 16 B)

template <int MF, int NFC, int PHASE>
__global__ __launch_bounds__(kThreads) void ffn_decode_bf16(
    const uint16_t* __restrict__ A, int K, const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
    int Ncols, const int4* __restrict__ tiles, const int* __restrict__ ntiles, uint16_t* __restrict__ out) {
  constexpr int NF = PHASE == 1 ? 2 * NFC : NFC;
  constexpr int BN = kWaves * 16 * NFC;
  constexpr int BM = 16 * MF;
  constexpr int U = kDecodeKC / 32;
  constexpr int VPR = kDecodeKC / 8;                       // uint4 per staged row
  constexpr int APT = (BM * VPR + kThreads - 1) / kThreads; // uint4 staged per thread
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kDecodeStride];

  const int nch = (Ncols + BN - 1) / BN;
  const int tile = blockIdx.x / nch;
  if (tile >= *ntiles) return;
  const int4 td = tiles[tile];
  const int row0 = td.y, rows = td.z, e = td.w;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int l16 = lane & 15, q = lane >> 4;
  const int col0 = (blockIdx.x % nch) * BN + wave * 16 * NFC;
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
      bf16x8 a[MF];
#pragma unroll
      for (int i = 0; i < MF; ++i)
        a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&as[(16 * i + l16) * kDecodeStride + 32 * u + 8 * q]));
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], __builtin_bit_cast(bf16x8, b[u][j]), acc[i][j], 0, 0, 0);
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

// ---- fp32 phase kernel (VALU, fp32 accumulation) --------------------------------
// One thread per output column, all rows of a 16-row tile.
template <int PHASE>
__global__ __launch_bounds__(kThreads) void ffn_phase_f32(const float* __restrict__ A, int K,
                                                          const float* __restrict__ W0, const float* __restrict__ W1,
                                                          int Ncols, const int4* __restrict__ tiles,
                                                          const int* __restrict__ ntiles, float* __restrict__ out) {
  constexpr int BM = 16;
  __shared__ float As[BM * 64];
  const int tile_id = blockIdx.x;
  if (tile_id >= *ntiles) return;
  const int4 td = tiles[tile_id];
  const int row0 = td.y, rows = td.z, e = td.w;
  const int n = blockIdx.y * kThreads + threadIdx.x;
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

struct Layout {
  int BM, max_tiles;
  bool stream;
  size_t tiles_off, ntiles_off, a_off, total;
};

// Rows per m-tile from the average group size (the host never sees the real
// group sizes): small groups stream weights (decode), large ones use LDS tiles.
int pick_mf(int n_rows, int G) {
  const int avg = G > 0 ? n_rows / G : n_rows;
  if (avg <= 8) return 1;
  if (avg <= 24) return 2;
  return 4;
}

bool use_stream(int n_rows, int G) { return G > 0 && n_rows / G <= 48; }

Layout layout(int n_rows, int E, int n_shared, int nseg, int d, int I, int bf16) {
  (void)d;
  Layout L;
  const int G = nseg * E + n_shared;
  L.stream = bf16 && use_stream(n_rows, G);
  L.BM = bf16 ? 16 * pick_mf(n_rows, G) : 16;
  L.max_tiles = (n_rows + L.BM - 1) / L.BM + G;
  L.tiles_off = 0;
  L.ntiles_off = ((static_cast<size_t>(L.max_tiles) * 16) + 255) / 256 * 256;
  L.a_off = L.ntiles_off + 256;
  const size_t a_bytes = static_cast<size_t>(n_rows) * I * (bf16 ? 2 : 4);
  L.total = L.a_off + (a_bytes + 255) / 256 * 256;
  return L;
}


template <int MF>
void launch_tile_bf16(const FfnArgs& a, const Layout& L, const int4* tiles, const int* ntiles, uint16_t* abuf,
                      hipStream_t stream) {
  constexpr int NFC = 1;
  const int bn = kWaves * 16 * NFC;
  dim3 g1(L.max_tiles, (a.I + bn - 1) / bn);
  hipLaunchKernelGGL((ffn_phase_bf16<MF, NFC, 1>), g1, dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(a.x_sorted), a.d, static_cast<const uint16_t*>(a.w_gate),
                     static_cast<const uint16_t*>(a.w_up), a.I, tiles, ntiles, abuf);
  dim3 g2(L.max_tiles, (a.d + bn - 1) / bn);
  hipLaunchKernelGGL((ffn_phase_bf16<MF, NFC, 2>), g2, dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(abuf), a.I, static_cast<const uint16_t*>(a.w_down),
                     static_cast<const uint16_t*>(nullptr), a.d, tiles, ntiles, static_cast<uint16_t*>(a.h_sorted));
}

// Decode-kernel shape: 16-column blocks per wave in each phase (the down
// projection gives each wave two blocks so both phases stream two weight rows
// per lane).
constexpr int kDecodeNfc1 = 1;
constexpr int kDecodeNfc2 = 2;

template <int MF>
void launch_decode_bf16(const FfnArgs& a, const Layout& L, const int4* tiles, const int* ntiles, uint16_t* abuf,
                        hipStream_t stream) {
  const int bn1 = kWaves * 16 * kDecodeNfc1, bn2 = kWaves * 16 * kDecodeNfc2;
  const int nch1 = (a.I + bn1 - 1) / bn1, nch2 = (a.d + bn2 - 1) / bn2;
  hipLaunchKernelGGL((ffn_decode_bf16<MF, kDecodeNfc1, 1>), dim3(L.max_tiles * nch1), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(a.x_sorted), a.d, static_cast<const uint16_t*>(a.w_gate),
                     static_cast<const uint16_t*>(a.w_up), a.I, tiles, ntiles, abuf);
  hipLaunchKernelGGL((ffn_decode_bf16<MF, kDecodeNfc2, 2>), dim3(L.max_tiles * nch2), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(abuf), a.I, static_cast<const uint16_t*>(a.w_down),
                     static_cast<const uint16_t*>(nullptr), a.d, tiles, ntiles, static_cast<uint16_t*>(a.h_sorted));
}

}  // namespace

size_t ffn_workspace_bytes(int n_rows, int E, int n_shared, int nseg, int d, int I, int bf16) {
  return layout(n_rows, E, n_shared, nseg, d, I, bf16).total;
}

hipError_t launch_ffn(const FfnArgs& a, void* workspace, hipStream_t stream) {
  const Layout L = layout(a.n_rows, a.E, a.n_shared, a.nseg, a.d, a.I, a.bf16);
  char* ws = static_cast<char*>(workspace);
  int4* tiles = reinterpret_cast<int4*>(ws + L.tiles_off);
  int* ntiles = reinterpret_cast<int*>(ws + L.ntiles_off);
  const int G = a.nseg * a.E + a.n_shared;
  hipLaunchKernelGGL(ffn_plan, dim3(1), dim3(kPlanThreads), 0, stream, a.group_offsets, G, a.E, a.nseg, L.BM,
                     a.n_rows, L.max_tiles, tiles, ntiles);
  if (a.bf16) {
    uint16_t* abuf = reinterpret_cast<uint16_t*>(ws + L.a_off);
    if (L.stream) {
      switch (L.BM / 16) {
        case 1: launch_decode_bf16<1>(a, L, tiles, ntiles, abuf, stream); break;
        case 2: launch_decode_bf16<2>(a, L, tiles, ntiles, abuf, stream); break;
        default: launch_decode_bf16<4>(a, L, tiles, ntiles, abuf, stream); break;
      }
    } else {
      switch (L.BM / 16) {
        case 1: launch_tile_bf16<1>(a, L, tiles, ntiles, abuf, stream); break;
        case 2: launch_tile_bf16<2>(a, L, tiles, ntiles, abuf, stream); break;
        default: launch_tile_bf16<4>(a, L, tiles, ntiles, abuf, stream); break;
      }
    }
  } else {
    float* abuf = reinterpret_cast<float*>(ws + L.a_off);
    dim3 g1(L.max_tiles, (a.I + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(ffn_phase_f32<1>, g1, dim3(kThreads), 0, stream, static_cast<const float*>(a.x_sorted), a.d,
                       static_cast<const float*>(a.w_gate), static_cast<const float*>(a.w_up), a.I, tiles, ntiles,
                       abuf);
    dim3 g2(L.max_tiles, (a.d + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(ffn_phase_f32<2>, g2, dim3(kThreads), 0, stream, static_cast<const float*>(abuf), a.I,
                       static_cast<const float*>(a.w_down), static_cast<const float*>(nullptr), a.d, tiles, ntiles,
                       static_cast<float*>(a.h_sorted));
  }
  return hipGetLastError();
}

}  // namespace moe
