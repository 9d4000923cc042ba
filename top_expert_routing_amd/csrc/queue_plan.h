// Tile order of the persistent single-launch expert FFN (ExpertPlex page,
// "Adaptive Persistent Kernels (APK)": expert work cut into tiles that
// resident workers take from a device-side queue, urgent decode tiles ahead of
// the rest, so a decode tile waits at most for the tiles already running).
//
// Plain index arithmetic shared by the GPU kernel and by a host-side checker:
// nothing here touches memory other than the arrays passed in.
//
// Sequences.  Sequence s is expert s.  With a priority segment (nseg == 2) a
// routed expert's rows are its priority group's rows A followed by its other
// group's rows B, tiled as one sequence A ++ B, so the expert's weights stream
// once for both; the units (m-tiles of bm rows) holding a row of A are its
// priority units.  A shared expert (s >= E) is its one group; without a
// priority segment every sequence is its one group.  Phase 1 (gate/up +
// SwiGLU) cuts the I columns into nch1 chunks, phase 2 (down projection) the d
// columns into nch2 chunks.
//
// Queues.  Chunk j of sequence s in phase p goes to queue
// (s * nch_p + j) mod nq, with all of that chunk's units, so the units that
// share a weight slab run from one queue (one XCD's L2 when the hardware deals
// a queue's blocks to one XCD) and a large expert's chunks spread over every
// queue.  Queue q's tiles, in pop order:
//   [P1: phase 1 of priority units][R1 head: the first `lag` phase-1 tiles of
//   the other units][P2: phase 2 of priority units][R1 tail][R2: phase 2 of
//   the other units]
// and inside each part sequence by sequence, chunk by chunk, unit by unit.
// A phase-2 tile of unit u needs the phase-1 tiles of u from every queue.
// Each queue lists every phase-1 tile it holds before any phase-2 tile of the
// same part, and all P1 tiles are at the front of their queues, so a
// waited-for tile has always been popped, or will be popped by a block of its
// queue that is not waiting (see queue_check in the tests).
#pragma once

#ifdef __HIPCC__
#define MOE_HD __host__ __device__ __forceinline__
#else
#define MOE_HD inline
#endif

namespace moe {
namespace qplan {

struct Shape {
  int E, S, nseg, n_rows;
  int bm;                   // unit rows
  int nch1, nch2;           // column chunks per phase
  int nq, lag;
  MOE_HD int nseq() const { return E + S; }
};

MOE_HD int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Row ranges of sequence s from the group offsets (clamped into [0, n_rows]).
struct SeqRows {
  int a0, na, b0, nb;       // A = [a0, a0 + na), B = [b0, b0 + nb)
  int prio;                 // rows of A that are priority rows (0 or na)
};

MOE_HD SeqRows seq_rows(const Shape& p, const int* offs, int s) {
  auto lo = [&](int i) { return clampi(offs[i], 0, p.n_rows); };
  SeqRows r;
  int ga = s;                                    // group of range A
  if (p.nseg == 2) ga = s < p.E ? s : p.E + s;   // shared expert s >= E is group 2E + (s - E)
  r.a0 = lo(ga);
  r.na = lo(ga + 1) - r.a0;
  if (r.na < 0) r.na = 0;
  r.b0 = r.a0 + r.na;
  r.nb = 0;
  r.prio = 0;
  if (p.nseg == 2 && s < p.E) {
    r.b0 = lo(p.E + s);
    r.nb = lo(p.E + s + 1) - r.b0;
    if (r.nb < 0) r.nb = 0;
    r.prio = r.na;
  }
  return r;
}

// Units of a sequence and how many of them are priority units.
struct SeqUnits {
  int units, tp;
};

MOE_HD SeqUnits seq_units(const Shape& p, const SeqRows& r) {
  SeqUnits u;
  u.units = (r.na + r.nb + p.bm - 1) / p.bm;
  u.tp = (r.prio + p.bm - 1) / p.bm;
  return u;
}

// Chunks of sequence s that queue q holds in a phase with nch chunks:
// j = first, first + nq, ... < nch.
MOE_HD int first_chunk(int s, int nch, int q, int nq) {
  const long long v = (static_cast<long long>(q) - static_cast<long long>(s) * nch) % nq;
  return static_cast<int>(v < 0 ? v + nq : v);
}
MOE_HD int chunks_in_queue(int first, int nch, int nq) { return first < nch ? (nch - 1 - first) / nq + 1 : 0; }

// Tile counts of sequence s in queue q: priority and other units, per phase.
struct SeqCounts {
  int p1, r1, p2, r2;
};

MOE_HD SeqCounts seq_counts(const Shape& p, int s, const SeqUnits& u, int q) {
  const int c1 = chunks_in_queue(first_chunk(s, p.nch1, q, p.nq), p.nch1, p.nq);
  const int c2 = chunks_in_queue(first_chunk(s, p.nch2, q, p.nq), p.nch2, p.nq);
  return SeqCounts{u.tp * c1, (u.units - u.tp) * c1, u.tp * c2, (u.units - u.tp) * c2};
}

// Queue q's part sizes (sums of seq_counts over the sequences).
struct QueueParts {
  int s1, s3, s2, s4;       // P1, R1, P2, R2 tile counts
  int s3a;                  // R1 tiles ahead of P2
  MOE_HD int total() const { return s1 + s3 + s2 + s4; }
};

MOE_HD QueueParts queue_parts(const Shape& p, const SeqCounts& sum) {
  QueueParts qp{sum.p1, sum.r1, sum.p2, sum.r2, 0};
  qp.s3a = qp.s3 < p.lag ? qp.s3 : p.lag;
  return qp;
}

// Pop position t of a queue -> (phase, priority part or not, index in that
// part's list).
struct Slot {
  int phase, prio, i;
};

MOE_HD Slot slot_of(const QueueParts& qp, int t) {
  if (t < qp.s1) return Slot{1, 1, t};
  t -= qp.s1;
  if (t < qp.s3a) return Slot{1, 0, t};
  t -= qp.s3a;
  if (t < qp.s2) return Slot{2, 1, t};
  t -= qp.s2;
  if (t < qp.s3 - qp.s3a) return Slot{1, 0, qp.s3a + t};
  t -= qp.s3 - qp.s3a;
  return Slot{2, 0, t};
}

// Last index g in [0, n) with pre[g] <= i (pre non-decreasing, pre[0] == 0).
MOE_HD int last_le(const int* pre, int n, int i) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= i) lo = mid; else hi = mid;
  }
  return lo;
}

// A decoded tile: sequence, chunk, unit within the sequence and its global
// unit id (fu[s] + mt), and its rows: tile row r < split is sorted row
// row0 + r, a later one row1 + (r - split).
struct Tile {
  int phase, prio, seq, chunk, mt, unit;
  int row0, rows, split, row1;
};

// `pre` is the exclusive prefix (over sequences, nseq + 1 entries) of this
// queue's tile counts for the slot's phase and part; `fu` the exclusive prefix
// of units over sequences.
MOE_HD Tile decode_tile(const Shape& p, const int* offs, const int* pre, const int* fu, int q, Slot sl) {
  const int ns = p.nseq();
  const int s = last_le(pre, ns, sl.i);
  const SeqRows r = seq_rows(p, offs, s);
  const SeqUnits u = seq_units(p, r);
  const int nch = sl.phase == 1 ? p.nch1 : p.nch2;
  const int nu = sl.prio ? u.tp : u.units - u.tp;      // units of this part (> 0 here)
  const int local = sl.i - pre[s];
  Tile t;
  t.phase = sl.phase;
  t.prio = sl.prio;
  t.seq = s;
  t.chunk = first_chunk(s, nch, q, p.nq) + p.nq * (local / nu);
  t.mt = (sl.prio ? 0 : u.tp) + local % nu;
  t.unit = fu[s] + t.mt;
  const int a = t.mt * p.bm;                            // first row of the unit in A ++ B
  const int rows = r.na + r.nb - a;
  t.rows = rows < p.bm ? rows : p.bm;
  t.row0 = r.a0 + a;
  t.split = clampi(r.na - a, 0, t.rows);
  t.row1 = r.b0 + (a > r.na ? a - r.na : 0);
  return t;
}

}  // namespace qplan
}  // namespace moe
