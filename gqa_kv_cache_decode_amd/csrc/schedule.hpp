// The static split of a decode step's work over persistent workgroups, as
// integer arithmetic shared by the device kernels and host-side checks.
//
// The work of one step is a sequence of segments, one per (sequence s, KV
// head group grp), ordered by s then grp; segment (s, grp) holds the
// tiles_of(L_s) 32-position tiles of sequence s (L_s its attended length).
// Tiles are grouped into schedule units of UT tiles (a segment's last unit
// may be short), and every non-empty segment is preceded by `lead` empty
// units that stand for the cost of opening a piece there. With T units in
// all and P' = min(P, T) workgroups taking part, workgroup p < P' takes the
// units [floor(p T / P'), floor((p + 1) T / P')). A workgroup's range is a
// run of pieces, the maximal runs of real units inside one segment; p0 and
// p1 are the first and the last workgroup holding real units of a piece's
// segment (p0 == p1: the segment is whole in one range).
#pragma once

#include <hip/hip_runtime.h>

namespace gqa {
namespace sched {

constexpr int kTilePositions = 32;

__host__ __device__ inline int tiles_of(int L) { return (L + kTilePositions - 1) / kTilePositions; }

// Real units of a segment of L positions.
template <int UT>
__host__ __device__ inline int units_of(int L) {
  return (L + kTilePositions * UT - 1) / (kTilePositions * UT);
}

// Units a segment occupies in the schedule: its real units and, when it has
// any, the lead units ahead of it.
template <int UT>
__host__ __device__ inline long long seg_units(int L, int lead) {
  const int nu = units_of<UT>(L);
  return nu > 0 ? nu + lead : 0;
}

// Workgroup owning unit u when T units are split over P workgroups as
// [floor(p T / P), floor((p + 1) T / P)): the largest p with floor(p T / P) <= u.
__host__ __device__ inline int owner_of(long long u, long long T, int P) {
  return int(((u + 1) * P + T - 1) / T) - 1;
}
__host__ __device__ inline long long range_begin(int p, long long T, int P) { return (long long)p * T / P; }

// Where a workgroup is in its range.
struct Cursor {
  long long total;     // units in all (T)
  long long u, u_end;  // the rest of the range
  long long seq_base;  // first unit of sequence s
  int s;               // sequence holding unit u
  int parts;           // workgroups taking part (P')
};

struct Piece {
  int s, grp, L;
  int tile_begin, tile_end;  // tiles [tile_begin, tile_end) of the segment
  int p0, p1;
};

// The next piece of the range; false once the range is done. len(s) gives
// the attended length of sequence s (< b).
template <int UT, typename LenFn>
__host__ __device__ inline bool next_piece(LenFn len, int b, int ngroups, int lead, Cursor& c, Piece& pc) {
  while (c.u < c.u_end) {
    int L = len(c.s);
    long long seq = (long long)ngroups * seg_units<UT>(L, lead);
    while (c.u >= c.seq_base + seq && c.s + 1 < b) {  // skip to the sequence holding u
      c.seq_base += seq;
      ++c.s;
      L = len(c.s);
      seq = (long long)ngroups * seg_units<UT>(L, lead);
    }
    const int nu = units_of<UT>(L);
    const int sl = nu + lead;
    const long long within = c.u - c.seq_base;
    const int grp = int(within / sl);
    const int ub = int(within - (long long)grp * sl);
    const long long remain = c.u_end - c.u;
    const long long seg_left = sl - ub;
    const int ue = ub + int(remain < seg_left ? remain : seg_left);
    c.u += ue - ub;
    const int rb = (ub > lead ? ub : lead) - lead;  // real units [rb, re) of the segment
    const int re = ue - lead;
    if (re <= rb) continue;  // only the segment's leading empty units
    const int nt = tiles_of(L);
    pc.s = c.s;
    pc.L = L;
    pc.grp = grp;
    pc.tile_begin = rb * UT;
    pc.tile_end = re * UT < nt ? re * UT : nt;
    const long long seg_u0 = c.seq_base + (long long)grp * sl + lead;  // first real unit
    pc.p0 = owner_of(seg_u0, c.total, c.parts);
    pc.p1 = owner_of(seg_u0 + nu - 1, c.total, c.parts);
    return true;
  }
  return false;
}

// The cursor of workgroup wg from the sequence-level unit counts (the
// kernels compute the same sums with a wave-wide prefix scan).
template <int UT, typename LenFn>
__host__ __device__ inline Cursor locate_serial(LenFn len, int b, int ngroups, int lead, int P, int wg) {
  Cursor c;
  long long total = 0;
  for (int s = 0; s < b; ++s) total += (long long)ngroups * seg_units<UT>(len(s), lead);
  c.total = total;
  c.parts = total < P ? int(total) : P;
  const bool takes_part = wg < c.parts;
  const int parts_nz = c.parts > 0 ? c.parts : 1;
  c.u = takes_part ? range_begin(wg, total, parts_nz) : 0;
  c.u_end = takes_part ? range_begin(wg + 1, total, parts_nz) : 0;
  c.s = b;
  c.seq_base = total;
  long long base = 0;
  for (int s = 0; s < b; ++s) {
    const long long v = (long long)ngroups * seg_units<UT>(len(s), lead);
    if (takes_part && v > 0 && base <= c.u && c.u < base + v) {
      c.s = s;
      c.seq_base = base;
      break;
    }
    base += v;
  }
  return c;
}

}  // namespace sched
}  // namespace gqa
