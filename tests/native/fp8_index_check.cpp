// Host-side walk of every block of the FP8-weight FFN's two launches (the
// decode-shaped kernel ffn_decode_fp8w), built from the same index code the
// kernel uses (top_expert_routing_amd/csrc/item_plan.h: work-item lookup and
// code addresses).  For the launch geometry the library picks (16 * MF-row
// tiles, K chunks of KC, eight waves of 16 * NFC columns) it checks that every
// block's item is valid, that every code, scale, token-row and output access
// lies inside its buffer, and that every output element of both phases is
// written exactly once.
//
// Input (stdin): d I E S nseg n_rows n_x MF packed has_rows, then G + 1 group
// offsets, then (has_rows) n_rows row-list entries.
// Prints "ok blocks=<n>" or "FAIL <reason>" (exit status 1).
#include <cstdio>
#include <vector>

#include "../../top_expert_routing_amd/csrc/item_plan.h"

using namespace moe;

static int fail(const char* why, long long a = 0, long long b = 0) {
  std::printf("FAIL %s %lld %lld\n", why, a, b);
  return 1;
}

static int kc_of(int MF) { return MF == 1 ? 512 : MF == 2 ? 384 : 256; }

int main() {
  int d, I, E, S, nseg, n_rows, n_x, MF, packed, has_rows;
  if (std::scanf("%d %d %d %d %d %d %d %d %d %d", &d, &I, &E, &S, &nseg, &n_rows, &n_x, &MF, &packed, &has_rows) != 10)
    return fail("bad header");
  const int G = nseg * E + S;
  std::vector<int> offs(G + 1), rowlist;
  for (auto& v : offs)
    if (std::scanf("%d", &v) != 1) return fail("bad offsets");
  if (has_rows) {
    rowlist.resize(n_rows);
    for (auto& v : rowlist)
      if (std::scanf("%d", &v) != 1) return fail("bad row list");
  }
  const int BM = 16 * MF, KC = kc_of(MF), U = KC / 64, VPR = KC / 8, NT = 512;
  const int APT = (BM * VPR + NT - 1) / NT;
  const int max_tiles = (n_rows + BM - 1) / BM + G;
  long long blocks_total = 0;
  for (int phase = 1; phase <= 2; ++phase) {
    const int K = phase == 1 ? d : I, Ncols = phase == 1 ? I : d, NFC = phase == 1 ? 1 : 2;
    const int NF = phase == 1 ? 2 * NFC : NFC, BN = 8 * 16 * NFC;
    const long long a_rows = phase == 1 ? (has_rows ? n_x : n_rows) : n_rows;
    const unsigned long long code_bytes = static_cast<unsigned long long>(E + S) * Ncols * K;
    const long long nch = (Ncols + BN - 1) / BN;
    const int grid = item_grid(max_tiles, static_cast<int>(nch));
    const int nchunks = (K + KC - 1) / KC;
    std::vector<unsigned char> written(static_cast<size_t>(n_rows) * (Ncols / 4), 0);
    for (int b = 0; b < grid; ++b) {
      const int x = b % kXcds, slot = b / kXcds;
      Item it{0, 0, 0, 0, 0, 0};
      int t = 0;
      for (int g = 0; g < G; ++g) {
        const GroupRows r = group_rows(offs.data(), n_rows, E, nseg, BM, g);
        const int n = group_items(r, g, static_cast<int>(nch), x);
        if (slot >= t && slot < t + n) it = group_item(r, g, static_cast<int>(nch), x, slot - t, BM, E, nseg);
        t += n;
      }
      if (it.rows == 0) continue;
      ++blocks_total;
      if (it.rows < 0 || it.rows > BM) return fail("item rows", b, it.rows);
      if (it.expert < 0 || it.expert >= E + S) return fail("item expert", b, it.expert);
      if (it.chunk < 0 || it.chunk >= nch) return fail("item chunk", b, it.chunk);
      for (int r = 0; r < it.rows; ++r)
        if (it.row(r) < 0 || it.row(r) >= n_rows) return fail("item row", b, it.row(r));
      const int e = it.expert;
      for (int w = 0; w < 8; ++w)
        for (int lane = 0; lane < 64; ++lane) {
          const int l16 = lane & 15, q = lane >> 4, tid = w * 64 + lane;
          const int col0 = it.chunk * BN + w * 16 * NFC;
          // weight codes
          for (int j = 0; j < NF; ++j) {
            int n = col0 + (j % NFC) * 16 + l16;
            n = n < Ncols - 1 ? n : Ncols - 1;
            for (int c = 0; c < nchunks; ++c)
              for (int u = 0; u < U; ++u) {
                const int kk = c * KC + 64 * u + 16 * q;
                if (kk >= K) continue;
                const unsigned long long off = fp8_code_offset(e, n, K, Ncols, lane, c * KC + 64 * u, packed != 0);
                if (off + 16 > code_bytes) return fail("code load out of range", b, static_cast<long long>(off));
              }
          }
          // token rows (A)
          for (int s = 0; s < APT; ++s) {
            const int idx = tid + s * NT;
            const int r = idx / VPR;
            if (idx >= BM * VPR || r >= it.rows) continue;
            const int sorted = it.row(r);
            long long arow = sorted;
            if (phase == 1 && has_rows) {
              const int v = rowlist[sorted];
              arow = v < 0 ? 0 : (v > n_x - 1 ? n_x - 1 : v);
            }
            for (int c = 0; c < nchunks; ++c) {
              const long long k = static_cast<long long>(c) * KC + (idx % VPR) * 8;
              if (k >= K) continue;
              if ((arow * K + k) * 2 + 16 > a_rows * K * 2) return fail("token-row load out of range", b, arow);
            }
          }
          // scales and outputs
          for (int i = 0; i < MF; ++i) {
            const int m = 16 * i + l16;
            if (m >= it.rows) continue;
            for (int j = 0; j < NFC; ++j) {
              const int n = col0 + j * 16 + 4 * q;
              if (n >= Ncols) continue;
              const long long so = static_cast<long long>(e) * Ncols + n;
              if ((so + 4) * 4 > static_cast<long long>(E + S) * Ncols * 4) return fail("scale load out of range", b, so);
              const long long o = static_cast<long long>(it.row(m)) * Ncols + n;
              if ((o + 4) * 2 > static_cast<long long>(n_rows) * Ncols * 2) return fail("store out of range", b, o);
              if (written[static_cast<size_t>(o / 4)]++) return fail("output written twice", it.row(m), n);
            }
          }
        }
    }
    for (size_t i = 0; i < written.size(); ++i)
      if (written[i] != 1) return fail("output element not written", static_cast<long long>(i / (Ncols / 4)), phase);
  }
  std::printf("ok blocks=%lld\n", blocks_total);
  return 0;
}
