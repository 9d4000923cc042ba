// Work items of the one-tile and decode-shaped FFN kernels: (m-tile of a group,
// column chunk), derived from the group offsets alone.  Plain index arithmetic
// shared by the GPU kernels (block_find_item scans it block-wide) and by a
// host-side checker that walks every block of a launch.
//
// The (group g, column chunk j) pairs are dealt to the 8 XCDs in turn: pair
// g * nch + j goes to XCD (g * nch + j) mod 8 with all of its m-tiles, and an
// XCD takes its pairs in group, chunk, m-tile order.  Workgroups are dealt to
// the XCDs round-robin (blockIdx mod 8), so block b runs item b / 8 of XCD
// b mod 8's list.
#pragma once

#ifndef MOE_HD
#ifdef __HIPCC__
#define MOE_HD __host__ __device__ __forceinline__
#else
#define MOE_HD inline
#endif
#endif

namespace moe {

constexpr int kXcds = 8;                    // MI355X: 8 XCDs, workgroups dealt round-robin

// A tile's rows: tile row r < split is sorted row row0 + r, a later one is
// row1 + (r - split) (two ranges when a priority group and the same expert's
// other rows share a tile; one range otherwise, split == rows).
struct Item {
  int row0, rows, expert, chunk;   // rows == 0: no work for this block
  int split, row1;
  MOE_HD int row(int r) const { return r < split ? row0 + r : row1 + (r - split); }
};

MOE_HD Item contiguous_item(int row0, int rows, int expert, int chunk) {
  return Item{row0, rows, expert, chunk, rows, row0 + rows};
}

// Column chunks of group g that XCD x holds: j = first, first + 8, ... < nch.
MOE_HD int xcd_first_chunk(int g, int nch, int x) {
  return static_cast<int>((static_cast<long long>(x) - static_cast<long long>(g) * nch) & (kXcds - 1));
}
MOE_HD int xcd_chunks(int first, int nch) { return first < nch ? (nch - 1 - first) / kXcds + 1 : 0; }

// Expert behind group g: routed groups seg*E + e, then the shared experts.
MOE_HD int group_expert(int g, int E, int nseg) { return g < nseg * E ? g % E : E + (g - nseg * E); }

// The rows a group's tiles cover: `na` rows from row `a0`, then `nb` rows from
// row `b0`, cut into m-tiles of BM; the group owns tiles [t0, t0 + nt).
struct GroupRows {
  int a0, na, b0, nb, t0, nt;
};

// With a priority segment (nseg == 2), expert e's priority rows P and its
// other rows R are tiled as one sequence P ++ R: group e (priority segment)
// owns the tiles that hold a row of P - so its first tile carries the first
// rows of R too, and the expert's weights stream once for both when R is
// small - and group E + e owns the remaining tiles.  Every priority row is
// still in the priority part of the list.  Otherwise a group is its own rows.
// Offsets are clamped into [0, n_rows].
MOE_HD GroupRows group_rows(const int* offs, int n_rows, int E, int nseg, int BM, int g) {
  auto lo = [&](int i) { const int v = offs[i]; return v < 0 ? 0 : (v > n_rows ? n_rows : v); };
  auto pos = [](int v) { return v < 0 ? 0 : v; };
  GroupRows r;
  if (nseg == 2 && g < 2 * E) {
    const int e = g < E ? g : g - E;
    r.a0 = lo(e);
    r.na = pos(lo(e + 1) - r.a0);
    r.b0 = lo(E + e);
    r.nb = pos(lo(E + e + 1) - r.b0);
    const int tp = (r.na + BM - 1) / BM;
    r.t0 = g < E ? 0 : tp;
    r.nt = g < E ? tp : (r.na + r.nb + BM - 1) / BM - tp;
  } else {
    r.a0 = lo(g);
    r.na = pos(lo(g + 1) - r.a0);
    r.b0 = r.a0 + r.na;
    r.nb = 0;
    r.t0 = 0;
    r.nt = (r.na + BM - 1) / BM;
  }
  return r;
}

// Items group g contributes to XCD x's list.
MOE_HD int group_items(const GroupRows& r, int g, int nch, int x) {
  return r.nt * xcd_chunks(xcd_first_chunk(g, nch, x), nch);
}

// The `local`-th of those items (0 <= local < group_items).
MOE_HD Item group_item(const GroupRows& r, int g, int nch, int x, int local, int BM, int E, int nseg) {
  const int j = xcd_first_chunk(g, nch, x) + kXcds * (local / r.nt);
  const int a = (r.t0 + local % r.nt) * BM;                  // first row of the tile in the sequence
  const int left = r.na + r.nb - a;
  const int rows = left < BM ? left : BM;
  const int sp = r.na - a;
  const int split = sp < 0 ? 0 : (sp > rows ? rows : sp);
  return Item{r.a0 + a, rows, group_expert(g, E, nseg), j, split, r.b0 + (a > r.na ? a - r.na : 0)};
}

// Grid size that covers every possible item of a call: XCD x holds at most
// ceil(nch / 8) chunks of each group, so at most max_tiles * ceil(nch / 8)
// items.
MOE_HD int item_grid(int max_tiles, int nch) {
  const long long per_xcd = static_cast<long long>(max_tiles) * ((nch + kXcds - 1) / kXcds);
  return static_cast<int>(per_xcd * kXcds);
}

// FP8 decode kernel: byte offset in a code array [E+S][Ncols][K] (row-major,
// or pre-packed in 16-row x 64-code blocks) of the 16 codes that lane `lane`
// (lane = 16 q + l16) of the wave owning weight row n loads for the 64-wide
// K-step starting at kk0 (a multiple of 64): codes kk0 + 16 q .. + 15 of row n.
// The offset is that of K position 0 plus fp8_code_step(kk0).
MOE_HD unsigned long long fp8_code_step(int kk0, bool packed) {
  return packed ? static_cast<unsigned long long>(kk0) * 16 : static_cast<unsigned long long>(kk0);
}
MOE_HD unsigned long long fp8_code_offset(int e, int n, int K, int Ncols, int lane, int kk0, bool packed) {
  const unsigned long long wstride = static_cast<unsigned long long>(Ncols) * K;
  const unsigned long long base = static_cast<unsigned long long>(e) * wstride;
  return (packed ? base + static_cast<unsigned long long>(n / 16) * (K / 64) * 1024 + lane * 16
                 : base + static_cast<unsigned long long>(n) * K + 16 * (lane >> 4)) +
         fp8_code_step(kk0, packed);
}

}  // namespace moe
