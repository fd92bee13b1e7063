// Host driver of the schedule arithmetic the decode kernels use
// (gqa_kv_cache_decode_amd/csrc/schedule.hpp), for the CPU schedule tests:
// every piece of every workgroup's range, as the kernels walk them.
#include "schedule.hpp"

namespace {

template <int UT>
int walk(const int* lens, int b, int ngroups, int lead, int P, int* out, int max_out) {
  auto len = [lens](int s) { return lens[s]; };
  int n = 0;
  for (int wg = 0; wg < P; ++wg) {
    gqa::sched::Cursor c = gqa::sched::locate_serial<UT>(len, b, ngroups, lead, P, wg);
    gqa::sched::Piece pc;
    int k = 0;
    while (gqa::sched::next_piece<UT>(len, b, ngroups, lead, c, pc)) {
      if (n < max_out) {
        int* o = out + 10 * n;
        o[0] = wg;
        o[1] = k;
        o[2] = pc.s;
        o[3] = pc.grp;
        o[4] = pc.tile_begin;
        o[5] = pc.tile_end;
        o[6] = pc.p0;
        o[7] = pc.p1;
        o[8] = c.u < c.u_end ? 1 : 0;  // units of the range left after this piece
        o[9] = c.parts;
      }
      ++n;
      ++k;
    }
  }
  return n;
}

}  // namespace

// unit_tiles 1 (the stream kernel) or 4 (the unit kernels); returns the
// number of pieces (rows of 10 ints written to out, at most max_out).
extern "C" int sched_pieces(int unit_tiles, const int* lens, int b, int ngroups, int lead, int P, int* out,
                            int max_out) {
  return unit_tiles == 1 ? walk<1>(lens, b, ngroups, lead, P, out, max_out)
                         : walk<4>(lens, b, ngroups, lead, P, out, max_out);
}
