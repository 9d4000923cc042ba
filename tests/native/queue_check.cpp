// Host-side check of the persistent FFN queue's tile order, built from the
// same header the GPU kernel includes (top_expert_routing_amd/csrc/queue_plan.h).
//
// Input (stdin, whitespace separated):
//   E S nseg n_rows bm nch1 nch2 nq lag units_cap
//   G+1 group offsets
// Checks, for every queue and pop position:
//   * every (phase, unit, chunk) of every unit appears exactly once over all
//     queues (phase 1: chunk < nch1, phase 2: chunk < nch2);
//   * the units of a sequence cover its rows A ++ B exactly once, in order,
//     and every tile row lies in [0, n_rows);
//   * unit ids and flag indices stay below the capacity the host allocates
//     (units_cap * nch1);
//   * with ONE block per queue (the hardest case: a waiting block stalls its
//     whole queue) processing pops in order, where a phase-1 tile completes
//     when popped and a phase-2 tile only once every phase-1 tile of its unit
//     has completed, every queue drains: no wait can stall on a tile that is
//     never popped.
// Prints "ok units=<n> tiles=<n>" or "FAIL <reason>" (exit status 1).
#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <tuple>
#include <vector>

#include "../../top_expert_routing_amd/csrc/queue_plan.h"

using namespace moe::qplan;

static int fail(const char* why, long long a = 0, long long b = 0) {
  std::printf("FAIL %s %lld %lld\n", why, a, b);
  return 1;
}

int main() {
  Shape p{};
  int units_cap = 0;
  if (std::scanf("%d %d %d %d %d %d %d %d %d %d", &p.E, &p.S, &p.nseg, &p.n_rows, &p.bm, &p.nch1, &p.nch2, &p.nq,
                 &p.lag, &units_cap) != 10)
    return fail("bad header");
  if (p.bm < 1 || p.nch1 < 1 || p.nch2 < 1 || p.nq < 1 || p.lag < 0) return fail("bad shape");
  const int G = p.nseg * p.E + p.S;
  std::vector<int> offs(G + 1);
  for (int i = 0; i <= G; ++i)
    if (std::scanf("%d", &offs[i]) != 1) return fail("bad offsets");
  const int ns = p.nseq();

  // units per sequence, exclusive prefix fu
  std::vector<SeqRows> rows(ns);
  std::vector<SeqUnits> su(ns);
  std::vector<int> fu(ns + 1, 0);
  for (int s = 0; s < ns; ++s) {
    rows[s] = seq_rows(p, offs.data(), s);
    su[s] = seq_units(p, rows[s]);
    fu[s + 1] = fu[s] + su[s].units;
  }
  const int units = fu[ns];
  if (units > units_cap) return fail("units above the host capacity", units, units_cap);
  // every sorted row belongs to exactly one sequence range
  std::vector<int> row_seen(p.n_rows, 0);
  for (int s = 0; s < ns; ++s) {
    for (int i = 0; i < rows[s].na; ++i) row_seen[rows[s].a0 + i]++;
    for (int i = 0; i < rows[s].nb; ++i) row_seen[rows[s].b0 + i]++;
  }
  for (int n = 0; n < p.n_rows; ++n)
    if (row_seen[n] != 1) return fail("sorted row not in exactly one sequence", n, row_seen[n]);

  // enumerate every queue
  struct Pop { int phase, unit, chunk, prio; };
  const int nqueues = p.nq;
  std::vector<std::vector<Pop>> qlist(nqueues);
  std::map<std::tuple<int, int, int>, int> seen;          // (phase, unit, chunk) -> count
  std::vector<std::vector<int>> unit_rows(units);         // rows of each unit (from its phase-1 chunk 0 tile)
  long long tiles = 0;
  for (int q = 0; q < nqueues; ++q) {
    std::vector<int> pre[4];                              // P1, R1, P2, R2 prefixes
    for (auto& v : pre) v.assign(ns + 1, 0);
    SeqCounts sum{0, 0, 0, 0};
    for (int s = 0; s < ns; ++s) {
      const SeqCounts c = seq_counts(p, s, su[s], q);
      pre[0][s + 1] = pre[0][s] + c.p1;
      pre[1][s + 1] = pre[1][s] + c.r1;
      pre[2][s + 1] = pre[2][s] + c.p2;
      pre[3][s + 1] = pre[3][s] + c.r2;
      sum.p1 += c.p1; sum.r1 += c.r1; sum.p2 += c.p2; sum.r2 += c.r2;
    }
    const QueueParts qp = queue_parts(p, sum);
    for (int t = 0; t < qp.total(); ++t) {
      const Slot sl = slot_of(qp, t);
      const int* pr = pre[(sl.phase == 1 ? 0 : 2) + (sl.prio ? 0 : 1)].data();
      const Tile tl = decode_tile(p, offs.data(), pr, fu.data(), q, sl);
      const int nch = tl.phase == 1 ? p.nch1 : p.nch2;
      if (tl.chunk < 0 || tl.chunk >= nch) return fail("chunk out of range", tl.chunk, nch);
      if (tl.unit < 0 || tl.unit >= units) return fail("unit out of range", tl.unit, units);
      if (tl.rows <= 0 || tl.rows > p.bm) return fail("tile rows", tl.rows, p.bm);
      if (tl.split < 0 || tl.split > tl.rows) return fail("split", tl.split, tl.rows);
      if (static_cast<long long>(tl.unit) * p.nch1 + tl.chunk >= static_cast<long long>(units_cap) * p.nch1)
        return fail("flag index above capacity", tl.unit, tl.chunk);
      const bool is_prio_unit = tl.mt < su[tl.seq].tp;
      if (is_prio_unit != (tl.prio != 0)) return fail("priority part holds a wrong unit", tl.unit, tl.prio);
      std::vector<int> rr;
      for (int r = 0; r < tl.rows; ++r) {
        const int n = r < tl.split ? tl.row0 + r : tl.row1 + (r - tl.split);
        if (n < 0 || n >= p.n_rows) return fail("tile row out of range", n, p.n_rows);
        rr.push_back(n);
      }
      if (tl.phase == 1 && tl.chunk == 0) unit_rows[tl.unit] = rr;
      if (++seen[{tl.phase, tl.unit, tl.chunk}] != 1) return fail("tile listed twice", tl.unit, tl.chunk);
      qlist[q].push_back(Pop{tl.phase, tl.unit, tl.chunk, tl.prio});
      ++tiles;
    }
  }
  // every unit's every chunk, both phases, exactly once
  for (int s = 0; s < ns; ++s)
    for (int mt = 0; mt < su[s].units; ++mt) {
      const int u = fu[s] + mt;
      for (int j = 0; j < p.nch1; ++j)
        if (seen[{1, u, j}] != 1) return fail("phase-1 tile missing", u, j);
      for (int j = 0; j < p.nch2; ++j)
        if (seen[{2, u, j}] != 1) return fail("phase-2 tile missing", u, j);
    }
  if (static_cast<long long>(seen.size()) != tiles) return fail("stray tiles", seen.size(), tiles);
  // units cover their sequence's rows A ++ B in order, exactly once
  for (int s = 0; s < ns; ++s) {
    std::vector<int> want, got;
    for (int i = 0; i < rows[s].na; ++i) want.push_back(rows[s].a0 + i);
    for (int i = 0; i < rows[s].nb; ++i) want.push_back(rows[s].b0 + i);
    for (int mt = 0; mt < su[s].units; ++mt)
      for (int n : unit_rows[fu[s] + mt]) got.push_back(n);
    if (want != got) return fail("units do not tile their sequence", s, static_cast<long long>(got.size()));
  }
  // one block per queue, pops in order
  std::vector<int> done1(units, 0), need1(units, 0);
  for (int s = 0; s < ns; ++s)
    for (int mt = 0; mt < su[s].units; ++mt) need1[fu[s] + mt] = p.nch1;
  std::vector<size_t> head(nqueues, 0);
  for (bool progress = true; progress;) {
    progress = false;
    for (int q = 0; q < nqueues; ++q) {
      while (head[q] < qlist[q].size()) {
        const Pop& x = qlist[q][head[q]];
        if (x.phase == 1) {
          done1[x.unit]++;
        } else if (done1[x.unit] < need1[x.unit]) {
          break;                      // this queue's only block waits here
        }
        ++head[q];
        progress = true;
      }
    }
  }
  for (int q = 0; q < nqueues; ++q)
    if (head[q] != qlist[q].size()) return fail("queue stalls on a wait that never ends", q, head[q]);
  std::printf("ok units=%d tiles=%lld\n", units, tiles);
  return 0;
}
