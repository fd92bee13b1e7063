// Matrix-core decode attention for up to 64 query heads per KV head (one,
// two or four 16-column MFMA blocks), bf16 K/V/q, d_k = d_v = 128, at most 64
// sequences: the Llama-3-70B- and Qwen2.5-7B-shaped GQA steps and the
// 32-head MQA ones with one query token per sequence, and causal calls with
// n query tokens per sequence whose n * G "virtual heads" fit in 64 (each
// token's heads see the cache and the new positions up to its own; MQA
// review §2.3, batched form with its mask). Same result as the other decode
// kernels (MQA review §2.1 per query head over the cache of §2.4 / §3;
// contiguous head groups of the TF2 GQA lesson); the per-tile arithmetic is
// the one of decode_matrix.hip (scores K·Q^T and output P·V on
// v_mfma_f32_16x16x32_bf16, base-2 softmax).
//
// What differs is how a workgroup walks its work, shaped by the measured
// timeline of the earlier schedule (per-workgroup clock stamps on the
// Llama-3-70B shape): the bulk of the stream ran at the memory system's
// rate, and the time was lost at the start (lengths, then query rows, then
// the first tile) and at the end, where the waves of one workgroup finished
// their statically dealt tiles up to ~13 µs apart (the compute unit serves
// its waves unevenly) and a barrier-bound merge and publish followed.
//
// * The static split of the (sequence, KV head) segments over the persistent
//   workgroups is balanced to one 32-position tile (16 KiB), not four.
// * Inside a workgroup, the streaming waves (seven with one head block, six
//   with two or four) take the range's tiles one at a time from an LDS
//   counter, so a wave that is served faster takes more tiles and all
//   finish together. Each tile's split-softmax state (max m, sum of
//   weights l, unnormalised output o) is computed from scratch, so it does
//   not depend on which wave computed it.
// * A folding wave per block of 16 heads (per 32 heads with four blocks)
//   folds the tile states in tile order out of an LDS ring (m = max, o and
//   l rescaled by 2^(m_k - m)), which fixes the arithmetic: results are bit
//   for bit the same whichever wave took which tile. It also writes,
//   publishes or merges each finished piece, so the streaming waves never
//   stop for that.
// * A tile's K/V loads are issued before the query rows it needs.
// * Fused step: a tile holding appended positions first stores their rows
//   into the cache. The grown lengths can be written as soon as every
//   workgroup has read the old ones, which all do at their start. The
//   folding wave of each workgroup counts it out right after that read on
//   one of 16 counters, and the last of each group on one more, so no more
//   than 16 atomics meet on one address; it waits for those results before
//   its first tile state arrives, and none waits at the end of the launch.
//
// Split segments (a segment whose tiles fall in the ranges of several
// workgroups, its "parts") are merged by the part that counts in last, with
// its own state still in registers. A part counts itself in on the
// segment's ticket (agent-scope atomic) a few tiles before it has folded its
// last one, so the round trip is hidden; a part that does not get the last
// ticket, once its last tile is folded, stores its state in its partial slot
// (SC1 stores, which bypass the non-coherent caches), waits for them, and
// raises the slot's ready flag. The last part, once its own tiles are
// folded, waits for the other parts' flags (each of those has counted in,
// so it is running and has only its own tiles and stores left; none waits
// for the merger, so the wait ends, and it is bounded all the same), reads
// their states (SC1 loads), merges them in part order and writes the output
// rows, then re-zeroes the ticket and the flags. Heavily split segments are
// instead left to a second launch (merge_partials_kernel).
#include <atomic>

#include "gqa_internal.hpp"

namespace gqa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kWaves = 8;
constexpr int kBlockThreads = kWaves * 64;
constexpr int kBlockHeads = 16;     // query heads of one MFMA column block
constexpr int kRow = kD + 4;        // LDS row stride (floats), padded against bank conflicts
// Tile states in the LDS ring with NB column blocks of heads (NB = 1, 2, 4:
// up to 16, 32, 64 heads per KV head); each way about 135 KB of LDS.
template <int NB>
constexpr int ring_slots() { return NB == 1 ? 16 : (NB == 2 ? 8 : 4); }
// Folding waves by head blocks: one per block of 16 heads for up to 32
// heads, one per 32 heads for 64 (so that six waves stream, not four).
template <int NB>
constexpr int folders() { return NB == 4 ? 2 : NB; }
constexpr int kCountTiles = 3;      // tiles before a piece's end at which it counts in on its ticket
constexpr int kFlagSpins = 1 << 22; // bound of the wait for another part's ready flag
// Parts of a segment whose states the merge holds in registers at once, by
// columns per lane.
template <int NCH>
constexpr int fast_slots() { return NCH == 16 ? 1 : (NCH == 8 ? 2 : (NCH == 4 ? 5 : 9)); }
// Ring slots the folding wave reads in one round, by columns per lane.
template <int NCH>
constexpr int fold_batch() { return NCH == 16 ? 1 : (NCH == 8 ? 2 : 4); }
constexpr int kCountGroups = 16;    // first-level counters of the fused step's length update
constexpr int kCountStride = 32;    // ints between counters (128 bytes)
// Spread merge: words of the stamp region, and the codes of its slot flags
// (a flag's high word; its low word is the generation that wrote it).
constexpr int kGenWord = 0;       // generation of the last launch
constexpr int kStartedWord = 32;  // generation whose workgroups have all started
constexpr unsigned kSpreadPublished = 0;  // state published; who merges its slice is not decided yet
constexpr unsigned kSpreadMerging = 1;    // state published; its part merges its own slice of heads
constexpr unsigned kSpreadOrphan = 2;     // state published; its slice is left to the workgroup that started last
constexpr unsigned kSpreadNone = 3;       // no partial state in this slot
constexpr int kStartSpins = 64;           // bound of a part's wait for every workgroup to have started
constexpr int kSweepPerThread = 2 * kMaxWorkgroups * kFlagBlocks / kBlockThreads;  // flags a thread polls, at most

__device__ __forceinline__ u32x4 ld16(const uint16_t* ptr) { return *reinterpret_cast<const u32x4*>(ptr); }
__device__ __forceinline__ void st16(uint16_t* ptr, u32x4 v) { *reinterpret_cast<u32x4*>(ptr) = v; }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int E>
__device__ __forceinline__ bf16x8 v_transpose(const u32x4* vr) {
  u32x4 a;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t x = vr[2 * k][E / 2];
    const uint32_t y = vr[2 * k + 1][E / 2];
    if constexpr ((E & 1) == 0) a[k] = (x & 0xffffu) | (y << 16);
    else a[k] = (x >> 16) | (y & 0xffff0000u);
  }
  return as_bf16x8(a);
}

// One 32-position tile in registers: K rows as the score MFMA's A operand
// (k[sg * 4 + ks]: row 16 sg + n16, dims 32 ks + 8 q4 .. +7), V rows
// v[r] = row 4 q4 + r (r < 4) or 16 + 4 q4 + r - 4 (dims 8 n16 .. +7): the
// positions this lane's k-slots of the value MFMA weigh (as in
// decode_matrix.hip).
struct Tile {
  u32x4 k[8];
  u32x4 v[8];
};

// Issue the loads of a tile whose rows start at kb / vb, rows < nvalid
// valid. Each half tile (16 rows) of K and of V is read through a buffer
// resource that covers exactly its valid rows: the hardware's range check
// (on the per-lane offset plus the instruction's constant offset, which
// stay below 4 KiB here) returns zero for the rows past them, with no
// per-row test, and nothing past the tile's valid rows is touched. Every
// address is one per-lane 32-bit offset plus a constant. Loads are
// non-temporal: each K/V byte is used once.
constexpr int kCpolStream = 2;  // NT
constexpr int kRowBytes = kD * int(sizeof(uint16_t));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t half_rsrc(const uint16_t* base, int half, int nvalid) {
  const int rows = nvalid - 16 * half;
  const int bytes = rows <= 0 ? 0 : (rows >= 16 ? 16 : rows) * kRowBytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base) + size_t(16 * half) * kD, 0, bytes,
                                           kBufferWord3);
}
__device__ __forceinline__ u32x4 tile_ld(__amdgpu_buffer_rsrc_t r, int voff, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + off, 0, kCpolStream));
}
__device__ __forceinline__ void load_tile(Tile& t, const uint16_t* kb, const uint16_t* vb, int nvalid, int n16,
                                          int q4) {
  // K row 16 sg + n16 (row n16 of half sg), dims 32 ks + 8 q4 .. +7
  const int ko = n16 * kRowBytes + q4 * 16;
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {
    const __amdgpu_buffer_rsrc_t rk = half_rsrc(kb, sg, nvalid);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) t.k[sg * 4 + ks] = tile_ld(rk, ko, ks * 64);
  }
  // V row 4 q4 + r (r < 4) or 16 + 4 q4 + r - 4, dims 8 n16 .. +7
  const int vo = 4 * q4 * kRowBytes + n16 * 16;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const __amdgpu_buffer_rsrc_t rv = half_rsrc(vb, hf, nvalid);
#pragma unroll
    for (int r = 0; r < 4; ++r) t.v[4 * hf + r] = tile_ld(rv, vo, r * kRowBytes);
  }
}

// op over the four 16-lane rows of the wave (lanes n, n + 16, n + 32,
// n + 48), the same value in all four: rows 0 and 1 and rows 2 and 3 are
// combined through the row-pair swap, then the two halves through the
// half swap (each a register exchange between lanes, no LDS round trip), as
// op(op(r0, r1), op(r2, r3)) for the symmetric ops used here.
template <typename Op>
__device__ __forceinline__ float across_rows(float x, Op op) {
  // (the pair's elements are copied to scalars before the bit casts: a cast
  // of a vector element in place reads element 0)
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // {r0 r0 r2 r2}, {r1 r1 r3 r3}
  const unsigned a0 = a[0], a1 = a[1];
  const float y = op(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
  const unsigned v = __builtin_bit_cast(unsigned, y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // {lo lo}, {hi hi}
  const unsigned b0 = b[0], b1 = b[1];
  return op(__builtin_bit_cast(float, b0), __builtin_bit_cast(float, b1));
}

// The split-softmax state of one tile, from scratch, for NB column blocks of
// 16 heads: per head m = the tile's largest scaled logit (base 2), l = sum
// of its weights 2^(s - m) (rounded to bf16, as applied), o = their
// weighted sum of V rows. Lane (n16, q4) holds head 16 b + n16 of block b:
// o[b][e][i] = dim 32 q4 + 8 i + e; m and l are the same in the head's four
// lanes. Unless FULL, the rows of block b at or past lim[b] are masked
// (lim[b] <= the tile's valid rows; below them only for a causal
// multi-token call). The K rows and the transposed V operands are shared by
// the blocks.
template <bool FULL, int NB>
__device__ __forceinline__ void tile_state(f32x4 (&o)[NB][8], float (&m)[NB], float (&l)[NB],
                                           const bf16x8 (*qop)[4], const Tile& t, const int* lim, float sl2,
                                           int q4) {
  bf16x8 pk[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float sv[8];  // scores, unscaled when FULL, else scaled and masked
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
      f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.k[sg * 4 + ks]), qop[b][ks], sacc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * sg + 4 * q4 + i;
        if constexpr (FULL) sv[sg * 4 + i] = sacc[i];
        else sv[sg * 4 + i] = row < lim[b] ? sacc[i] * sl2 : kNegInf;
      }
    }
    // m: the largest scaled score. In a full tile it is found on the
    // unscaled scores (the largest for a positive scale, the smallest for a
    // negative one) and scaled once: a correctly rounded product keeps the
    // order, so this is the same value as the largest rounded product.
    float mx = sv[0];
    if (FULL && sl2 < 0.0f) {
#pragma unroll
      for (int k = 1; k < 8; ++k) mx = fminf(mx, sv[k]);
      mx = across_rows(mx, [](float x, float y) { return fminf(x, y); });
    } else {
#pragma unroll
      for (int k = 1; k < 8; ++k) mx = fmaxf(mx, sv[k]);
      mx = across_rows(mx, [](float x, float y) { return fmaxf(x, y); });
    }
    if constexpr (FULL) mx *= sl2;
    const float sub = (mx == kNegInf) ? 0.0f : mx;
    // weights 2^(s - m), rounded to bf16 in pairs (the value MFMA's operand);
    // the denominator sums the weights as rounded, in position order
    float psum = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
      float e0, e1;
      if constexpr (FULL) {
        e0 = fast_exp2(fmaf(sv[k], sl2, -sub));
        e1 = fast_exp2(fmaf(sv[k + 1], sl2, -sub));
      } else {
        e0 = fast_exp2(sv[k] - sub);
        e1 = fast_exp2(sv[k + 1] - sub);
      }
      const bf16x2 pr = __builtin_convertvector((f32x2){e0, e1}, bf16x2);
      pk[b][k] = pr[0];
      pk[b][k + 1] = pr[1];
      const uint32_t w = __builtin_bit_cast(uint32_t, pr);
      psum += __builtin_bit_cast(float, w << 16);
      psum += __builtin_bit_cast(float, w & 0xffff0000u);
    }
    psum = across_rows(psum, [](float x, float y) { return x + y; });
    m[b] = mx;
    l[b] = psum;
  }
#define GQA_PV(E)                                                                                       \
  {                                                                                                     \
    const bf16x8 vt = v_transpose<E>(t.v);                                                              \
    _Pragma("unroll") for (int b = 0; b < NB; ++b) o[b][E] =                                            \
        __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pk[b], f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);     \
  }
  GQA_PV(0) GQA_PV(1) GQA_PV(2) GQA_PV(3) GQA_PV(4) GQA_PV(5) GQA_PV(6) GQA_PV(7)
#undef GQA_PV
}

// The schedule (schedule.hpp) in single tiles: segments (s, j) ordered by s,
// then j, segment (s, j) preceded by `lead` empty tiles (the cost of
// opening a piece, so that a range starting just before a segment skips
// them), workgroup p < P' taking tiles [floor(p T / P'), floor((p + 1) T / P')).
using Range = sched::Cursor;
using StreamPiece = sched::Piece;

// Wave-uniform values computed through lane shuffles, made visibly uniform
// (scalar registers) for the compiler.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ long long uni(long long x) {
  const unsigned lo = __builtin_amdgcn_readfirstlane(unsigned(x & 0xffffffffll));
  const unsigned hi = __builtin_amdgcn_readfirstlane(unsigned((unsigned long long)x >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// Every lane of the wave: the workgroup's range from the lengths (lane s
// holds L_s; b <= 64); the sums of sched::locate_serial as a wave scan.
__device__ Range locate(const DecodeParams& p, int Lreg, int wg) {
  const int lane = threadIdx.x & 63;
  const long long v = lane < p.b ? (long long)p.g * sched::seg_units<1>(Lreg, p.seg_lead) : 0;
  const long long incl = wave_inclusive_scan(v);
  Range r;
  r.total = uni(__shfl(incl, 63, 64));
  r.parts = r.total < p.workgroups ? int(r.total) : p.workgroups;
  const bool takes_part = wg < r.parts;
  const int parts_nz = r.parts > 0 ? r.parts : 1;
  r.u = uni(takes_part ? sched::range_begin(wg, r.total, parts_nz) : 0);
  r.u_end = uni(takes_part ? sched::range_begin(wg + 1, r.total, parts_nz) : 0);
  const long long excl = incl - v;
  const unsigned long long hit = __ballot(lane < p.b && v > 0 && excl <= r.u && r.u < incl);
  const int src = hit ? __ffsll((long long)hit) - 1 : 0;
  r.s = uni(hit ? src : p.b);
  r.seq_base = uni(hit ? __shfl(excl, src, 64) : r.total);
  return r;
}

// Next piece of the range (lengths from the lane registers via shuffles).
__device__ __forceinline__ bool next_piece(const DecodeParams& p, Range& r, int Lreg, StreamPiece& pc) {
  return sched::next_piece<1>([Lreg](int s) { return uni(__shfl(Lreg, s, 64)); }, p.b, p.g, p.seg_lead, r, pc);
}

// Row in q and out of (virtual) head hh of KV group j of sequence s, GV
// heads per group: s * h + j * GV + hh for one query token per sequence;
// for a causal multi-token call virtual head hh is token hh / G's head
// j * G + hh mod G (head_row).
template <bool CAUSAL>
__device__ __forceinline__ size_t vrow(const DecodeParams& p, int s, int j, int GV, int hh) {
  if constexpr (CAUSAL) return head_row(p.n_tok, p.h, p.G, s, j * GV + hh);
  else return size_t(s) * p.h + size_t(j) * GV + hh;
}

// Byte offset of partial slot `slot` of workgroup `wg`.
__device__ __forceinline__ int slot_offset(const DecodeParams& p, int wg, int slot) {
  return (wg * 2 + slot) * p.slot_floats * int(sizeof(float));
}

// One step of the in-order merge of a segment's partial states: fold the
// state (m, l, o) of the next part into the running (run, den, acc). Every
// merge of a split segment in this kernel goes through this exact sequence,
// so its result does not depend on which workgroup or path performed it.
struct MergeWeights2 {
  float r, w, run;
};
__device__ __forceinline__ MergeWeights2 merge_weights2(float run, float m) {
  const float M = fmaxf(run, m);
  const float sub = (M == kNegInf) ? 0.0f : M;
  return {fast_exp2(run - sub), fast_exp2(m - sub), M};
}
__device__ __forceinline__ f32x4 merge_o(f32x4 acc, const MergeWeights2& mw, f32x4 o) {
  f32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = __builtin_fmaf(mw.w, o[e], acc[e] * mw.r);
  return out;
}
__device__ __forceinline__ float merge_l(float den, const MergeWeights2& mw, float l) {
  return __builtin_fmaf(mw.w, l, den * mw.r);
}
__device__ __forceinline__ uint2 to_bf16x4(f32x4 v) {
  uint2 pk;
  pk.x = uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16);
  pk.y = uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16);
  return pk;
}

// Counting the workgroups out after their read of the lengths (fused step)
// and of the launch generation (spread merge). Workgroup wg counts on
// first-level counter wg mod 16; the last of each group counts on the top
// counter; the last of those writes the lengths (fused step), publishes that
// every workgroup of this generation has started and takes the orphaned
// merges (spread merge), and re-zeroes all counters.
struct LenCount {
  // called by one wave of the workgroup after the workgroup barrier that
  // follows the read of lens (its values are in LDS by then). It waits for
  // each count's result right away: the folding wave that runs it has
  // nothing to fold until the first tile states arrive, well after both
  // round trips, and no atomic's result is left pending into the fold loop
  // (a result pending across the loop's back edge made the compiler wait
  // for every outstanding memory access, stores included, at each piece).
  template <bool SPREAD>
  __device__ static void run(const DecodeParams& p, const int* s_lens, int wg, bool write_lens, unsigned stamp,
                             int* s_sweep) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // keep the count after the read of lens
    const int lane = threadIdx.x & 63;
    const int P = int(gridDim.x);
    int v = 0;
    if (lane == 0)
      v = __hip_atomic_fetch_add(p.ws_done + kCountStride * (1 + wg % kCountGroups), 1, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    v = __builtin_amdgcn_readfirstlane(v);
    const int grp = wg % kCountGroups;
    const int members = (P - grp + kCountGroups - 1) / kCountGroups;
    if (v != members - 1) return;
    // the last of its group counts the group out on the top counter
    int t = 0;
    if (lane == 0) t = __hip_atomic_fetch_add(p.ws_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    t = __builtin_amdgcn_readfirstlane(t);
    const int groups = P < kCountGroups ? P : kCountGroups;
    if (t != groups - 1) return;
    // the last of all: every workgroup has read the old lengths and the generation
    if (write_lens && lane < p.b) p.lens[lane] = s_lens[lane];  // attended length = grown length
    if (SPREAD && lane == 0) {
      __hip_atomic_store(p.ws_stamp + kGenWord, int(stamp), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.ws_stamp + kStartedWord, int(stamp), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *s_sweep = 1;
    }
    if (lane < groups)
      __hip_atomic_store(p.ws_done + kCountStride * (1 + lane), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane == 0) __hip_atomic_store(p.ws_done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};

// Ready flag of folding wave `half`'s heads in partial slot `slot` of workgroup `wg`
// (zero between calls).
__device__ __forceinline__ int* slot_flag(const DecodeParams& p, int wg, int slot, int half) {
  return p.ws_done + kFlagsOffset / sizeof(int) + (wg * 2 + slot) * kFlagBlocks + half;
}
// Spread merge: stamped flag of folding wave `half`'s heads in partial slot
// `slot` of workgroup `wg` (never reset), and its value for a generation and
// a code.
__device__ __forceinline__ unsigned long long* spread_flag(const DecodeParams& p, int wg, int slot, int half) {
  return reinterpret_cast<unsigned long long*>(p.ws_stamp + kStampFlagsOffset / sizeof(int)) +
         (wg * 2 + slot) * kFlagBlocks + half;
}
__device__ __forceinline__ unsigned long long flag_value(unsigned stamp, unsigned code) {
  return (static_cast<unsigned long long>(code) << 32) | stamp;
}

// The merging folding wave `half` waits until every other part of segment
// p0 .. p0 + n_slots - 1 has raised that wave's ready flag (each
// part has already taken its ticket, so it is running and has only its own
// tiles and stores left). The wait is bounded.
__device__ void wait_parts(const DecodeParams& p, int p0, int n_slots, int own, int half) {
  const int lane = threadIdx.x & 63;
  for (int q0 = 0; q0 < n_slots; q0 += 64) {
    const int q = q0 + lane;
    const bool need = q < n_slots && q != own;
    int* f = need ? slot_flag(p, p0 + q, q == 0 ? 1 : 0, half) : nullptr;
    for (int it = 0; it < kFlagSpins; ++it) {
      const bool ready = !need || __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
      if (__ballot(!ready) == 0) break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
}

// Merge of the parts of segment (s, j) in part order (slot 1 of p0, then
// slot 0 of p0 + 1 .. p0 + n_slots - 1), with part `own` taken from this
// wave's registers, up to B parts' loads in flight at a time; then the
// output rows. Lane layout as in fold_range, heads from h0.
template <int NCH, bool CAUSAL>
__device__ void merge_parts(const DecodeParams& p, int s, int j, int p0, int n_slots, int own, int h0,
                            const f32x4 (&own_o)[NCH], float own_m, float own_l) {
  constexpr int HP = (kD / 4) / NCH;
  constexpr int B = fast_slots<NCH>();
  const int lane = threadIdx.x & 63;
  const int G = p.gblk;
  const int hh = h0 + lane / HP;
  const int sub = lane % HP;
  if (hh >= G) return;
  const __amdgpu_buffer_rsrc_t rs = slots_rsrc(p);
  const int ml_off = G * kD * int(sizeof(float));
  float run = kNegInf, den = 0.0f;
  f32x4 res[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) res[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = 0; k0 < n_slots; k0 += B) {
    f32x4 o[B][NCH];
    float m[B], l[B];
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int k = k0 + q;
      if (k < n_slots && k != own) {
        const int sb = slot_offset(p, p0 + k, k == 0 ? 1 : 0);
#pragma unroll
        for (int i = 0; i < NCH; ++i) o[q][i] = coherent_load4(rs, sb + (hh * kD + 4 * (sub + HP * i)) * 4);
        m[q] = coherent_load1(rs, sb + ml_off + hh * 4);
        l[q] = coherent_load1(rs, sb + ml_off + (G + hh) * 4);
      }
    }
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int k = k0 + q;
      if (k < n_slots) {
        const bool mine = k == own;
        const MergeWeights2 mw = merge_weights2(run, mine ? own_m : m[q]);
#pragma unroll
        for (int i = 0; i < NCH; ++i) res[i] = merge_o(res[i], mw, mine ? own_o[i] : o[q][i]);
        den = merge_l(den, mw, mine ? own_l : l[q]);
        run = mw.run;
      }
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  uint16_t* out = static_cast<uint16_t*>(p.out) + vrow<CAUSAL>(p, s, j, G, hh) * kD;
#pragma unroll
  for (int i = 0; i < NCH; ++i) *reinterpret_cast<uint2*>(out + 4 * (sub + HP * i)) = to_bf16x4(res[i] * inv);
}

// A folding wave: fold the tile states of the workgroup's range in tile
// order for its heads and finish every piece for them (write them out,
// publish them or merge them). With NB = 2 there is one folding wave per
// block of 16 heads, with NB = 4 one per 32 heads, each working alone on
// its heads with its own ready flags; wave 0 of them also counts the
// workgroup out for the fused step's lengths and takes the piece tickets,
// and hands each ticket's result to the other through LDS (s_tk: value and
// piece number, 16 pieces deep; no folding wave is more than a ring's worth
// of tiles, hence of pieces, behind wave 0). Lane layout: HP = 32 / NCH
// lanes per head (NCH = 2, 4, 8, 16 for up to 4, 8, 16, 32 heads per
// wave); lane l of folding wave hb holds head (64 / HP) hb + l / HP and its
// four-dim columns c = (l mod HP) + HP i, i < NCH, so each lane weighs a
// single head per tile. The ring has ring_slots<NB>() slots of 16 NB heads;
// s_folded[hb] counts the tiles folding wave hb has folded.
template <int NCH, bool FUSED, int NB, bool CAUSAL, bool SPREAD>
__device__ void fold_range(const DecodeParams& p, const Range& range, int Lreg, int hb,
                           float (*s_o)[kBlockHeads * NB * kRow], float (*s_m)[kBlockHeads * NB],
                           float (*s_l)[kBlockHeads * NB], int* s_ready, int* s_folded, int (*s_tk)[16],
                           const int* s_lens, unsigned stamp, int* s_spread, int* s_sweep) {
  constexpr int HP = (kD / 4) / NCH;
  constexpr int R = fold_batch<NCH>();
  constexpr int kRing = ring_slots<NB>();
  const int wg = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int G = p.gblk;  // (virtual) heads per KV group
  const int h0 = (64 / HP) * hb;  // heads per folding wave: 64 / HP
  const int hh = h0 + lane / HP;
  const int sub = lane % HP;
  const bool active = hh < G;
  const bool lead = hb == 0;  // counts, takes tickets
  if ((FUSED || SPREAD) && lead) LenCount::run<SPREAD>(p, s_lens, wg, FUSED, stamp, s_sweep);
  Range it = range;
  StreamPiece pc;
  int k = 0;    // next range tile to fold
  int ord = 0;  // pieces finished so far
  int published = 0;  // spread merge: partial slots this wave has published (bits)
  for (; next_piece(p, it, Lreg, pc); ++ord) {
    const int n = pc.tile_end - pc.tile_begin;
    const int s = pc.s, j = pc.grp;
    const bool shared = pc.p0 != pc.p1;
    const bool inline_merge = shared && !p.merge_kernel && !SPREAD;
    const int n_slots = pc.p1 - pc.p0 + 1;
    const int own = wg - pc.p0;  // this workgroup's part of the segment
    int* ticket = p.ws_cnt + (size_t(s) * p.ngroups + j) * p.cnt_stride;
    // a few tiles before the end, count in on the segment's ticket: the part
    // that counts in last merges, the others publish at their end
    const int count_at = n > kCountTiles ? n - kCountTiles : 0;
    int t = 0;
    f32x4 acc[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float am = kNegInf, al = 0.0f;
    for (int e = 0; e < n;) {
      const int slot = k & (kRing - 1);
      while (__hip_atomic_load(&s_ready[slot], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != k)
        __builtin_amdgcn_s_sleep(1);
      // tile k is in; so may be the next few: take the run of them that is
      // ready (up to R, inside the piece) with one round of LDS reads, then
      // fold them one by one in tile order (the same arithmetic as one at a
      // time, so the result does not depend on how they were batched)
      int rd[R];
#pragma unroll
      for (int i = 1; i < R; ++i)
        rd[i] = __hip_atomic_load(&s_ready[(k + i) & (kRing - 1)], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
      int r = 1;
#pragma unroll
      for (int i = 1; i < R; ++i)
        if (r == i && e + i < n && rd[i] == k + i) r = i + 1;
      r = __builtin_amdgcn_readfirstlane(r);
      if (lead && inline_merge && lane == 0 && count_at >= e && count_at < e + r)
        t = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (active) {
        f32x4 ot[R][NCH];
        float mt[R], lt[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          if (i < r) {
            const int sl = (k + i) & (kRing - 1);
            const float* row = &s_o[sl][hh * kRow + 4 * sub];
#pragma unroll
            for (int c = 0; c < NCH; ++c) ot[i][c] = *reinterpret_cast<const f32x4*>(row + 4 * HP * c);
            mt[i] = s_m[sl][hh];
            lt[i] = s_l[sl][hh];
          }
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
          if (i < r) {
            // the same step as every merge of split states (2^(m_k - m) rescale)
            const MergeWeights2 mw = merge_weights2(am, mt[i]);
#pragma unroll
            for (int c = 0; c < NCH; ++c) acc[c] = merge_o(acc[c], mw, ot[i][c]);
            al = merge_l(al, mw, lt[i]);
            am = mw.run;
          }
        }
      }
      // every lane's reads of the slots are done before they are handed back
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
      e += r;
      k += r;
      if (lane == 0) __hip_atomic_store(&s_folded[hb], k, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    // the piece is complete
    if (!shared) {
      if (active) {
        uint16_t* out = static_cast<uint16_t*>(p.out) + vrow<CAUSAL>(p, s, j, G, hh) * kD;
        const float inv = al > 0.0f ? 1.0f / al : 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) *reinterpret_cast<uint2*>(out + 4 * (sub + HP * i)) = to_bf16x4(acc[i] * inv);
      }
      if (lead && p.merge_kernel && pc.tile_begin == 0 && lane == 0)
        p.seg_info[size_t(s) * p.ngroups + j] = make_int2(pc.p0, -1);
      continue;
    }
    if (inline_merge) {
      if (lead) {
        t = __builtin_amdgcn_readfirstlane(t);
        if (NB > 1 && lane == 0) {
          s_tk[0][ord & 15] = t;
          __hip_atomic_store(&s_tk[1][ord & 15], ord + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      } else {
        while (__hip_atomic_load(&s_tk[1][ord & 15], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != ord + 1)
          __builtin_amdgcn_s_sleep(1);
        t = __builtin_amdgcn_readfirstlane(s_tk[0][ord & 15]);
      }
    }
    if (inline_merge && t == n_slots - 1) {
      // the last part: merge once the others' states are in their slots, and
      // leave the ticket and their flags at zero
      wait_parts(p, pc.p0, n_slots, own, hb);
      merge_parts<NCH, CAUSAL>(p, s, j, pc.p0, n_slots, own, h0, acc, am, al);
      if (lane < n_slots && lane != own)
        __hip_atomic_store(slot_flag(p, pc.p0 + lane, lane == 0 ? 1 : 0, hb), 0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      if (lead && lane == 0) __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      continue;
    }
    // publish this part's state, then (inline and spread merges) its flag
    const __amdgpu_buffer_rsrc_t rs = slots_rsrc(p);
    const int ml_off = G * kD * int(sizeof(float));
    const int my_slot = wg == pc.p0 ? 1 : 0;
    const int slot_off = slot_offset(p, wg, my_slot);
    // spread merge: whether every workgroup of this launch has started, read
    // while the state is stored. If so, every part of the segment reaches its
    // end without waiting on anything, so this part may wait for them at the
    // end of the launch and merge its own slice of heads; if not yet, that is
    // decided at the end of the launch.
    int started = 0;
    if (SPREAD && lane == 0)
      started = __hip_atomic_load(p.ws_stamp + kStartedWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (active) {
#pragma unroll
      for (int i = 0; i < NCH; ++i)
        coherent_store4(rs, slot_off + (hh * kD + 4 * (sub + HP * i)) * int(sizeof(float)), acc[i]);
      if (sub == 0) {
        coherent_store1(rs, slot_off + ml_off + hh * 4, am);
        coherent_store1(rs, slot_off + ml_off + (G + hh) * 4, al);
      }
    }
    if (SPREAD) {
      wait_stores();
      const unsigned code =
          unsigned(__builtin_amdgcn_readfirstlane(started)) == stamp ? kSpreadMerging : kSpreadPublished;
      if (lane == 0) {
        __hip_atomic_store(spread_flag(p, wg, my_slot, hb), flag_value(stamp, code), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        int* job = s_spread + 8 * my_slot;  // the piece, for the end of the launch
        job[0] = s;
        job[1] = j;
        job[2] = pc.p0;
        job[3] = n_slots;
        job[4] = own;
        job[5 + hb] = int(code);
        job[7] = 1;
      }
      published |= 1 << my_slot;
    } else if (p.merge_kernel) {
      if (lead && pc.tile_begin == 0 && lane == 0) p.seg_info[size_t(s) * p.ngroups + j] = make_int2(pc.p0, pc.p1);
    } else {
      wait_stores();
      if (lane == 0)
        __hip_atomic_store(slot_flag(p, wg, my_slot, hb), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // spread merge: the slots this wave left empty are stamped too, so that the
  // workgroup that started last can tell when every part has published
  if (SPREAD && lane == 0) {
    for (int sl = 0; sl < 2; ++sl)
      if (!(published & (1 << sl)))
        __hip_atomic_store(spread_flag(p, wg, sl, hb), flag_value(stamp, kSpreadNone), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---- spread merge: at the end of the launch, every thread of the workgroup

__device__ __forceinline__ bool stamped(unsigned long long flag, unsigned stamp) {
  return unsigned(flag) == stamp;
}
__device__ __forceinline__ unsigned flag_code(unsigned long long flag) { return unsigned(flag >> 32); }

// Wave 0: wait until the n parts of a segment (partial slots of workgroups
// p0 .. p0 + n - 1) have stamped the flags of their NF folding waves with this
// generation. Only called once every workgroup of the generation has
// started: each part then reaches its end without waiting on anything, so
// the wait ends; it is bounded all the same.
template <int NF>
__device__ void wait_spread(const DecodeParams& p, int p0, int n, unsigned stamp) {
  constexpr int U = 4;  // flags per lane in one round of loads
  const int lane = threadIdx.x & 63;
  const int total = n * NF;
  for (int q0 = 0; q0 < total; q0 += 64 * U) {
    unsigned long long* f[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + 64 * u + lane;
      const int k = q / NF;
      f[u] = q < total ? spread_flag(p, p0 + k, k == 0 ? 1 : 0, q - k * NF) : nullptr;
    }
    for (int it = 0; it < kFlagSpins; ++it) {
      unsigned long long v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = f[u] ? __hip_atomic_load(f[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
      bool ready = true;
#pragma unroll
      for (int u = 0; u < U; ++u) ready = ready && (!f[u] || stamped(v[u], stamp));
      if (__ballot(!ready) == 0) break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
}

// Merge of heads list[0 .. cnt) of segment (s, j), whose n parts' states sit
// in the partial slots of workgroups p0 .. p0 + n - 1 (slot 1 of p0, slot 0
// of the others), and their output rows, by the whole workgroup. A head's
// arithmetic depends only on n, not on which workgroup merges it: its R =
// min(16, n) rows of 32 threads (R a power of two; 16 / R heads per pass)
// fold parts r, r + R, r + 2R, ... in order (row r, thread c: dims 4c ..
// 4c + 3, four parts' loads in flight), and the R row states are then folded
// in row order through LDS (buf: 16 x 32 f32x4, then 16 m and 16 l). Every
// fold is the step of the in-order merge above.
template <bool CAUSAL>
__device__ void merge_heads(const DecodeParams& p, int s, int j, int p0, int n, const int* list, int cnt,
                            float* buf) {
  const int tid = threadIdx.x;
  const int r16 = tid >> 5, c = tid & 31;
  int R = 1;
  while (2 * R <= n && 2 * R <= 16) R *= 2;
  const int per_pass = 16 / R;
  const int hs = r16 / R, rr = r16 - hs * R;
  const int G = p.gblk;
  const __amdgpu_buffer_rsrc_t rs = slots_rsrc(p);
  const int ml_off = G * kD * int(sizeof(float));
  for (int base = 0; base < cnt; base += per_pass) {
    const int hi = base + hs;
    const bool valid = hi < cnt;
    const int hh = valid ? list[hi] : 0;
    float run = kNegInf, den = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (valid) {
      for (int k0 = rr; k0 < n; k0 += 4 * R) {
        f32x4 o[4];
        float m[4], l[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int k = k0 + u * R;
          if (k < n) {
            const int sb = slot_offset(p, p0 + k, k == 0 ? 1 : 0);
            o[u] = coherent_load4(rs, sb + (hh * kD + 4 * c) * int(sizeof(float)));
            m[u] = coherent_load1(rs, sb + ml_off + hh * 4);
            l[u] = coherent_load1(rs, sb + ml_off + (G + hh) * 4);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (k0 + u * R < n) {
            const MergeWeights2 mw = merge_weights2(run, m[u]);
            acc = merge_o(acc, mw, o[u]);
            den = merge_l(den, mw, l[u]);
            run = mw.run;
          }
        }
      }
    }
    *reinterpret_cast<f32x4*>(buf + 4 * tid) = acc;
    if (c == 0) {
      buf[2048 + r16] = run;
      buf[2064 + r16] = den;
    }
    __syncthreads();
    if (valid && rr == 0) {
      float run2 = kNegInf, den2 = 0.0f;
      f32x4 res = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int r = 0; r < R; ++r) {
        const int row = hs * R + r;
        const MergeWeights2 mw = merge_weights2(run2, buf[2048 + row]);
        res = merge_o(res, mw, *reinterpret_cast<const f32x4*>(buf + 4 * (row * 32 + c)));
        den2 = merge_l(den2, mw, buf[2064 + row]);
        run2 = mw.run;
      }
      const float inv = den2 > 0.0f ? 1.0f / den2 : 0.0f;
      uint16_t* out = static_cast<uint16_t*>(p.out) + vrow<CAUSAL>(p, s, j, G, hh) * kD;
      *reinterpret_cast<uint2*>(out + 4 * c) = to_bf16x4(res * inv);
    }
    __syncthreads();
  }
}

// The end of a spread-merge launch. Each shared piece of this workgroup
// (s_spread: per partial slot the segment, its first part p0, its part count
// n, this part's index, the code of each folding wave's flag) has been
// published. A folding wave's heads whose flag is not decided yet wait a
// bounded time for every workgroup to have started: if they all have, they
// are this part's to merge (kSpreadMerging), else they are left to the
// workgroup that started last (kSpreadOrphan); the flag then says which.
// This part merges heads own, own + n, own + 2n, ... of the segment, those
// that are its to merge, once every part has stamped its flags. The
// workgroup that started last (s_sweep) then waits until every flag of the
// generation is stamped and decided, and merges the orphaned slices.
// buf: the free LDS ring.
template <int NB, bool CAUSAL>
__device__ void spread_end(const DecodeParams& p, int parts, int Lreg, unsigned stamp, int* s_spread,
                           const int* s_sweep, float* buf) {
  constexpr int NF = folders<NB>();
  constexpr int kFolderHeads = kBlockHeads * NB / NF;  // heads per folding wave
  int* list = reinterpret_cast<int*>(buf + 2080);      // heads to merge (up to 64)
  int* orph = reinterpret_cast<int*>(buf + 2176);      // count, then orphaned flags (workgroup, slot, wave)
  const int tid = threadIdx.x, w = tid >> 6;
  const int G = p.gblk;
  __syncthreads();  // every wave has published; the ring is free
  // undecided slices: wait (bounded) for every workgroup to have started
  bool undecided = false;
  for (int slot = 0; slot < 2; ++slot)
    for (int hb = 0; hb < NF; ++hb)
      undecided = undecided || (s_spread[8 * slot + 7] != 0 && s_spread[8 * slot + 5 + hb] == int(kSpreadPublished));
  if (undecided) {
    __syncthreads();  // every thread has read the codes before they change
    if (w == 0) {
      bool all_started = false;
      for (int it = 0; it < kStartSpins && !all_started; ++it) {
        int v = 0;
        if ((tid & 63) == 0)
          v = __hip_atomic_load(p.ws_stamp + kStartedWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        all_started = unsigned(__builtin_amdgcn_readfirstlane(v)) == stamp;
        if (!all_started) __builtin_amdgcn_s_sleep(8);
      }
      if (tid == 0) {
        const unsigned code = all_started ? kSpreadMerging : kSpreadOrphan;
        for (int slot = 0; slot < 2; ++slot)
          for (int hb = 0; hb < NF; ++hb)
            if (s_spread[8 * slot + 7] != 0 && s_spread[8 * slot + 5 + hb] == int(kSpreadPublished)) {
              s_spread[8 * slot + 5 + hb] = int(code);
              __hip_atomic_store(spread_flag(p, blockIdx.x, slot, hb), flag_value(stamp, code), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
            }
      }
    }
    __syncthreads();
  }
  for (int slot = 0; slot < 2; ++slot) {
    const int* job = s_spread + 8 * slot;
    if (job[7] == 0) continue;
    const int s = job[0], j = job[1], p0 = job[2], n = job[3], own = job[4];
    int cnt = 0;
    for (int hh = own; hh < G; hh += n)
      if (job[5 + hh / kFolderHeads] == int(kSpreadMerging)) {
        if (tid == 0) list[cnt] = hh;
        ++cnt;
      }
    if (cnt == 0) continue;
    if (w == 0) wait_spread<NF>(p, p0, n, stamp);
    __syncthreads();
    merge_heads<CAUSAL>(p, s, j, p0, n, list, cnt, buf);
  }
  if (*s_sweep == 0) return;
  // every workgroup of the generation has started: wait for all their flags
  // (one round of loads per thread), collect the orphaned slices
  const int nflags = parts * 2 * NF;
  if (tid == 0) orph[0] = 0;
  __syncthreads();
  unsigned long long v[kSweepPerThread];
  unsigned long long* f[kSweepPerThread];
#pragma unroll
  for (int u = 0; u < kSweepPerThread; ++u) {
    const int q = tid + u * kBlockThreads;
    const int wgx = q / (2 * NF), rem = q - wgx * (2 * NF);
    f[u] = q < nflags ? spread_flag(p, wgx, rem / NF, rem % NF) : nullptr;
    v[u] = f[u] ? __hip_atomic_load(f[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
  }
#pragma unroll
  for (int u = 0; u < kSweepPerThread; ++u) {
    if (f[u]) {
      for (int it = 0; it < kFlagSpins && !(stamped(v[u], stamp) && flag_code(v[u]) != kSpreadPublished); ++it) {
        __builtin_amdgcn_s_sleep(2);
        v[u] = __hip_atomic_load(f[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (flag_code(v[u]) == kSpreadOrphan) {
        const int pos = __hip_atomic_fetch_add(&orph[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        orph[1 + pos] = tid + u * kBlockThreads;
      }
    }
  }
  __syncthreads();
  const int norph = orph[0];
  for (int o = 0; o < norph; ++o) {
    const int q = orph[1 + o];
    const int wgx = q / (2 * NF), rem = q - wgx * (2 * NF);
    const int sl = rem / NF, hb = rem - sl * NF;
    // the orphan's piece: the shared piece of workgroup wgx's range in slot sl
    Range rx = locate(p, Lreg, wgx);
    StreamPiece pc;
    bool found = false;
    while (next_piece(p, rx, Lreg, pc))
      if (pc.p0 != pc.p1 && (wgx == pc.p0 ? 1 : 0) == sl) {
        found = true;
        break;
      }
    if (!found) continue;
    const int n = pc.p1 - pc.p0 + 1;
    int cnt = 0;
    for (int hh = wgx - pc.p0; hh < G; hh += n)
      if (hh / kFolderHeads == hb) {
        if (tid == 0) list[cnt] = hh;
        ++cnt;
      }
    if (cnt == 0) continue;
    __syncthreads();
    merge_heads<CAUSAL>(p, pc.s, pc.grp, pc.p0, n, list, cnt, buf);
  }
}

template <bool FUSED, bool PAGED, int NB, bool CAUSAL, bool SPREAD>
__global__ __launch_bounds__(kBlockThreads, 1) void decode_stream_kernel(DecodeParams p) {
  constexpr int kRing = ring_slots<NB>();
  constexpr int kHeads = kBlockHeads * NB;
  __shared__ __attribute__((aligned(16))) float s_o[kRing][kHeads * kRow];
  __shared__ float s_m[kRing][kHeads];
  __shared__ float s_l[kRing][kHeads];
  __shared__ int s_ready[kRing];  // range tile index whose state a ring slot holds (-1: none yet)
  __shared__ int s_lens[64];
  __shared__ int s_next;          // next range tile to hand out
  __shared__ int s_folded[folders<NB>()];  // range tiles folded so far, per folding wave
  __shared__ int s_tk[2][16];     // ticket results handed from block 0's folding wave to the others
  __shared__ int s_gen;           // spread merge: the generation of the last launch
  __shared__ int s_sweep;         // spread merge: this workgroup started last
  __shared__ int s_spread[16];    // spread merge: this workgroup's shared pieces, by partial slot
  constexpr int kStreamers = kWaves - folders<NB>();  // waves 0 .. kStreamers - 1 stream, the others fold

  const int wg = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n16 = lane & 15;
  const int q4 = lane >> 4;
  const int G = p.gblk;  // (virtual) heads per KV group
  const float sl2 = p.scale_log2;

  if (w == 0) s_lens[lane] = lane < p.b ? attended_len(p, lane) : 0;
  if (threadIdx.x < kRing) s_ready[threadIdx.x] = -1;
  if (threadIdx.x < folders<NB>()) s_folded[threadIdx.x] = 0;
  if (threadIdx.x < 16) s_tk[1][threadIdx.x] = 0;
  if (threadIdx.x < 16) s_spread[threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    s_next = 0;
    s_sweep = 0;
    s_gen = SPREAD ? __hip_atomic_load(p.ws_stamp + kGenWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
  }
  if (!FUSED) zero_empty_sequences<uint16_t, CAUSAL>(p, wg);
  __syncthreads();

  const int Lreg = s_lens[lane];
  const Range range = locate(p, Lreg, wg);
  // this launch's generation (spread merge); never zero, the value of zeroed flags
  const unsigned stamp = unsigned(s_gen) + 1u == 0u ? 1u : unsigned(s_gen) + 1u;

  if (w < kStreamers) {
    // ---- streaming wave: take tiles, leave their states in the ring
    Range it = range;
    StreamPiece pc;
    bool have = next_piece(p, it, Lreg, pc);
    long long kb = 0;             // range tiles before piece pc
    int q_seg = -1;               // segment whose query rows are in qop
    bf16x8 qop[NB][4];
    while (have) {
      int k = 0;
      if (lane == 0) k = __hip_atomic_fetch_add(&s_next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      k = __builtin_amdgcn_readfirstlane(k);
      while (have && k >= kb + (pc.tile_end - pc.tile_begin)) {
        kb += pc.tile_end - pc.tile_begin;
        have = next_piece(p, it, Lreg, pc);
      }
      if (!have) break;
      const int s = pc.s, j = pc.grp;
      const size_t kv_head = size_t(s) * p.g + j;
      const int tile = pc.tile_begin + int(k - kb);
      const int t0 = tile * kTile;
      const int nvalid = pc.L - t0;
      // fused step: the appended tokens are the segment's last p.fused
      // positions; a tile holding any of them stores their rows (token r of
      // sequence s from k_new / v_new [b][n][g][d]) into their cache slots,
      // waits for the stores, then reads the tile. Lanes l and l + 32 take
      // two consecutive positions, lanes 0-15 of each half the K row and
      // lanes 16-31 the V row; up to eight rows' loads are issued before the
      // first store, so that the rows cost one round trip, not one each.
      const int first_new = pc.L - p.fused;
      if (FUSED && t0 + kTile > first_new) {
        const int n_new = p.fused;
        const int pos0 = t0 > first_new ? t0 : first_new;
        const int pos_end = pc.L < t0 + kTile ? pc.L : t0 + kTile;
        const bool is_v = (lane & 16) != 0;
        const int col = 8 * (lane & 15);
        const uint16_t* src_base = static_cast<const uint16_t*>(is_v ? p.v_new : p.k_new);
        uint16_t* dst_base = static_cast<uint16_t*>(is_v ? p.v_cache : p.k_cache);
        constexpr int kRowBatch = 4;
        for (int base = pos0; base < pos_end; base += 2 * kRowBatch) {
          u32x4 row[kRowBatch];
#pragma unroll
          for (int i = 0; i < kRowBatch; ++i) {
            const int pos = base + 2 * i + (lane >> 5);
            if (pos < pos_end)
              row[i] = ld16(src_base + ((size_t(s) * n_new + (pos - first_new)) * p.g + j) * kD + col);
          }
#pragma unroll
          for (int i = 0; i < kRowBatch; ++i) {
            const int pos = base + 2 * i + (lane >> 5);
            if (pos < pos_end) st16(dst_base + kv_row<PAGED, true>(p.pg, p.g, p.cap, s, j, pos) * kD + col, row[i]);
          }
        }
        wait_stores();
      }
      const uint16_t* kbp;
      const uint16_t* vbp;
      if constexpr (PAGED) {
        const size_t row = kv_row<true, true>(p.pg, p.g, p.cap, s, j, t0);
        kbp = static_cast<const uint16_t*>(p.k_cache) + row * kD;
        vbp = static_cast<const uint16_t*>(p.v_cache) + row * kD;
      } else {
        kbp = static_cast<const uint16_t*>(p.k_cache) + (kv_head * p.cap + t0) * kD;
        vbp = static_cast<const uint16_t*>(p.v_cache) + (kv_head * p.cap + t0) * kD;
      }
      Tile t;
      load_tile(t, kbp, vbp, nvalid < kTile ? nvalid : kTile, n16, q4);
      const int seg = s * p.g + j;
      if (seg != q_seg) {
        // the group's query rows, after the tile's loads are on their way
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int head = kBlockHeads * b + n16;
          const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + vrow<CAUSAL>(p, s, j, G, head) * kD;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (head < G) v = ld16(qrow + ks * 32 + q4 * 8);
            qop[b][ks] = as_bf16x8(v);
          }
        }
        q_seg = seg;
      }
      // rows each head block sees: the tile's valid rows, and for a causal
      // multi-token call only those before its token's position (virtual
      // head v is token v / G_real, which sees n_tok - 1 - v / G_real fewer
      // of the last positions; padding heads as many as the last token)
      int lim[NB];
      bool full = nvalid >= kTile;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        lim[b] = nvalid < kTile ? nvalid : kTile;
        if constexpr (CAUSAL) {
          const int head = kBlockHeads * b + n16;
          const int hide = head < G ? p.n_tok - 1 - head / p.G : 0;
          const int seen = pc.L - t0 - hide;
          lim[b] = seen < lim[b] ? seen : lim[b];
        }
      }
      if constexpr (CAUSAL) full = full && pc.L - t0 - (p.n_tok - 1) >= kTile;
      // the state is computed and deposited in one pass for one or two head
      // blocks, in one pass per block for four (registers); the first pass
      // is computed before the wait for the slot, so that the wait overlaps it
      constexpr int BP = NB == 4 ? 1 : NB;
      const int slot = k & (kRing - 1);
#pragma unroll
      for (int bp = 0; bp < NB; bp += BP) {
        f32x4 o[BP][8];
        float m[BP], l[BP];
        if (full) tile_state<true, BP>(o, m, l, &qop[bp], t, &lim[bp], sl2, q4);
        else tile_state<false, BP>(o, m, l, &qop[bp], t, &lim[bp], sl2, q4);
        if (bp == 0) {
          // slot k mod kRing is free once tile k - kRing has been folded (by
          // every head block's folding wave)
          while (true) {
            int folded = __hip_atomic_load(&s_folded[0], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
            for (int f = 1; f < folders<NB>(); ++f) {
              const int ff = __hip_atomic_load(&s_folded[f], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
              folded = ff < folded ? ff : folded;
            }
            if (folded > k - kRing) break;
            __builtin_amdgcn_s_sleep(1);
          }
        }
#pragma unroll
        for (int b = 0; b < BP; ++b) {
          const int head = kBlockHeads * (bp + b) + n16;
          if (head < G) {
            float* row = &s_o[slot][head * kRow + 32 * q4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              *reinterpret_cast<f32x4*>(row + 8 * i) = f32x4{o[b][0][i], o[b][1][i], o[b][2][i], o[b][3][i]};
              *reinterpret_cast<f32x4*>(row + 8 * i + 4) = f32x4{o[b][4][i], o[b][5][i], o[b][6][i], o[b][7][i]};
            }
            if (q4 == 0) {
              s_m[slot][head] = m[b];
              s_l[slot][head] = l[b];
            }
          }
        }
      }
      // every lane's writes are done before the slot is marked
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
      if (lane == 0) __hip_atomic_store(&s_ready[slot], k, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  } else if constexpr (NB == 1) {
    // ---- folding waves (one per block of 16 heads, or per 32 with four
    // blocks; lane layout by the heads in use)
    if (G <= 4)
      fold_range<2, FUSED, NB, CAUSAL, SPREAD>(p, range, Lreg, 0, s_o, s_m, s_l, s_ready, s_folded, s_tk, s_lens, stamp,
                                       s_spread, &s_sweep);
    else if (G <= 8)
      fold_range<4, FUSED, NB, CAUSAL, SPREAD>(p, range, Lreg, 0, s_o, s_m, s_l, s_ready, s_folded, s_tk, s_lens, stamp,
                                       s_spread, &s_sweep);
    else
      fold_range<8, FUSED, NB, CAUSAL, SPREAD>(p, range, Lreg, 0, s_o, s_m, s_l, s_ready, s_folded, s_tk, s_lens, stamp,
                                       s_spread, &s_sweep);
  } else {
    // 16 heads per folding wave (NCH = 8) with two blocks, 32 (NCH = 16) with four
    fold_range<NB == 4 ? 16 : 8, FUSED, NB, CAUSAL, SPREAD>(p, range, Lreg, w - kStreamers, s_o, s_m, s_l, s_ready,
                                                    s_folded, s_tk, s_lens, stamp, s_spread, &s_sweep);
  }
  if constexpr (SPREAD) spread_end<NB, CAUSAL>(p, range.parts, Lreg, stamp, s_spread, &s_sweep, &s_o[0][0]);
}

template <bool FUSED, bool PAGED, bool CAUSAL, bool SPREAD>
void launch_merge(const DecodeParams& p, hipStream_t stream) {
  if (p.gblk <= kBlockHeads)
    hipLaunchKernelGGL((decode_stream_kernel<FUSED, PAGED, 1, CAUSAL, SPREAD>), dim3(p.workgroups),
                       dim3(kBlockThreads), 0, stream, p);
  else if (p.gblk <= 2 * kBlockHeads)
    hipLaunchKernelGGL((decode_stream_kernel<FUSED, PAGED, 2, CAUSAL, SPREAD>), dim3(p.workgroups),
                       dim3(kBlockThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_stream_kernel<FUSED, PAGED, 4, CAUSAL, SPREAD>), dim3(p.workgroups),
                       dim3(kBlockThreads), 0, stream, p);
}
// The spread merge is its own set of instances, so that the others compile
// as they would without it; it is requested through the contiguous
// one-token calls only (the host refuses it elsewhere).
template <bool FUSED, bool PAGED, bool CAUSAL>
void launch(const DecodeParams& p, hipStream_t stream) {
  if constexpr (!PAGED && !CAUSAL) {
    if (p.merge_spread) {
      launch_merge<FUSED, PAGED, CAUSAL, true>(p, stream);
      return;
    }
  }
  launch_merge<FUSED, PAGED, CAUSAL, false>(p, stream);
}

}  // namespace

hipError_t launch_decode_stream(const DecodeParams& p, hipStream_t stream) {
  const bool paged = p.pg.table != nullptr;
  if (p.n_tok > 1) {
    if (p.fused) paged ? launch<true, true, true>(p, stream) : launch<true, false, true>(p, stream);
    else paged ? launch<false, true, true>(p, stream) : launch<false, false, true>(p, stream);
  } else {
    if (p.fused) paged ? launch<true, true, false>(p, stream) : launch<true, false, false>(p, stream);
    else paged ? launch<false, true, false>(p, stream) : launch<false, false, false>(p, stream);
  }
  return hipGetLastError();
}

// Workgroups of the instance that fit on one compute unit (cached per
// process; the answer depends only on the kernel and the architecture).
int stream_workgroups_per_cu(bool fused, bool paged, int G) {
  static std::atomic<int> cached[12] = {};
  const int nb = G <= kBlockHeads ? 0 : (G <= 2 * kBlockHeads ? 1 : 2);
  const int k = (fused ? 1 : 0) + (paged ? 2 : 0) + 4 * nb;
  const int known = cached[k].load(std::memory_order_relaxed);
  if (known > 0) return known;
  int n = 0;
  hipError_t e;
  switch (k) {
    case 0: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<false, false, 1, false, false>, kBlockThreads, 0); break;
    case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<true, false, 1, false, false>, kBlockThreads, 0); break;
    case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<false, true, 1, false, false>, kBlockThreads, 0); break;
    case 3: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<true, true, 1, false, false>, kBlockThreads, 0); break;
    case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<false, false, 2, false, false>, kBlockThreads, 0); break;
    case 5: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<true, false, 2, false, false>, kBlockThreads, 0); break;
    case 6: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<false, true, 2, false, false>, kBlockThreads, 0); break;
    case 7: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<true, true, 2, false, false>, kBlockThreads, 0); break;
    case 8: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<false, false, 4, false, false>, kBlockThreads, 0); break;
    case 9: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<true, false, 4, false, false>, kBlockThreads, 0); break;
    case 10: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<false, true, 4, false, false>, kBlockThreads, 0); break;
    default: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<true, true, 4, false, false>, kBlockThreads, 0); break;
  }
  if (e != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 0;
  }
  cached[k].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace gqa
