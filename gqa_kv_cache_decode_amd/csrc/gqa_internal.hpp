// Internal declarations shared by the gfx950 kernels and the C-ABI shim.
//
// Work schedule (both decode kernels)
// -----------------------------------
// The attention of one decode step is cut into units of four 32-position
// tiles of one "segment" (sequence s, KV-head group grp); a segment's last
// unit may be short. Units are
// ordered (s, grp, unit). With T units in all and P' = min(P, T) of the P
// persistent workgroups taking part, workgroup p < P' takes the contiguous
// range [floor(p*T/P'), floor((p+1)*T/P')) (never empty), so every workgroup
// streams the same number of K/V bytes (within one unit) and all finish
// together. T depends on the device-side lengths, so each wave recomputes the
// schedule from lens at kernel start (a prefix sum over b).
//
// A workgroup's range is a run of "pieces": maximal runs of units inside one
// segment. Only its first and its last piece can be part of a segment shared
// with other workgroups; whole segments are written out directly. A shared
// piece leaves its split-softmax state (m, l, o) in one of the workgroup's
// two partial slots. Attention over a set of positions split into parts is
// recovered exactly from the parts' states: with M = max_k m_k, the output is
// sum_k 2^(m_k - M) o_k / sum_k 2^(m_k - M) l_k (the softmax of the MQA
// review, §2.1, written over a union of position sets). Either the last
// workgroup of the segment to arrive (an atomic ticket per segment) merges
// the slots, or, for shapes whose segments are split over many workgroups, a
// second launch (merge_partials_kernel) merges every shared segment with one
// workgroup per (segment, query head).
//
// Cross-workgroup visibility without cache-wide fences: on this multi-XCD
// part a device-scope release fence writes back a whole L2, which costs more
// than the attention itself. The partial states are therefore written with
// buffer stores that bypass the non-coherent caches (SC1), their completion
// is awaited (s_waitcnt vmcnt(0)) before the ticket's agent-scope atomic add,
// and the merging workgroup reads them with SC1 buffer loads. Only these
// accesses touch the shared data, so no L2 writeback or invalidate is needed.
//
// Workspace layout (caller-owned, see gqa_decode_workspace_size), from the
// start of the buffer:
//   [segment table] int2 [b * h]                              separate merge only
//   [slots]  float [kMaxWorkgroups][2][slot_floats]           slot = o[gb][d], m[gb], l[gb]
// and from its end (size rounded down to 256 bytes):
//   [tickets] int32, cnt_stride apart                         zero between calls
//   [done]   int32 counters and slot flags, kDoneBytes         zero between calls
//   [stamps] spread-merge generations and flags, last kStampBytes   zero before the first call
// slot_floats = gb*d + round_up(2*gb, 4), so every slot and its o block are
// 16-byte aligned. Each region starts on a 256-byte boundary.
//
// Cache layouts. Contiguous: K [b][g][cap][d_k], V [b][g][cap][d_v]. Paged:
// pools K [num_blocks][g][B][d_k], V [num_blocks][g][B][d_v] of blocks of B =
// 2^bs_log2 >= 32 positions, and a block table int32 [b][table_stride]:
// position t of sequence s lives in block table[s][t >> bs_log2] at row
// t & (B - 1). A 32-position tile never straddles two blocks, so the kernels
// look the block up once per tile; everything else is shared.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "schedule.hpp"

namespace gqa {

constexpr int kThreads = 256;  // workgroup size of the merge kernel (and of the 4-wave decode instances)
constexpr int kTile = 32;             // positions per wave step
constexpr int kUnitTiles = 4;         // tiles per schedule unit
constexpr int kMaxWorkgroups = 2048;  // persistent grid bound (workspace sizing)
constexpr int kMatrixMaxGroup = 64;   // query heads per KV head on the matrix path
constexpr int kVectorMaxBlock = 8;    // query heads per workgroup on the vector path

// Paged cache addressing (table == nullptr: contiguous [b][g][cap][d]).
struct PagedLayout {
  const int32_t* table;  // [b][table_stride] block ids
  int table_stride;
  int bs_log2;           // block of 2^bs_log2 positions
  int num_blocks;        // ids are clamped to [0, num_blocks)
};

struct AppendParams {
  void* k_cache;
  void* v_cache;
  const void* k_new;
  const void* v_new;
  int32_t* lens;
  int g, d_k, d_v, cap;
  PagedLayout pg;
  int n_tok;  // new tokens per sequence (k_new [b][n_tok][g][d_k])
};

struct DecodeParams {
  void* out;
  const void* q;
  void* k_cache;      // written only by the fused step (the new row)
  void* v_cache;
  int32_t* lens;      // written only by the fused step (+1, by the last workgroup)
  const void* k_new;  // fused step: the new token's rows [b][g][d]
  const void* v_new;
  int* ws_cnt;        // tickets, cnt_stride ints apart
  int* ws_done;       // fused step: workgroups finished (zero between calls)
  float* ws_slots;
  int b, h, g, G, d, cap;
  int max_len;        // bound of the attended lengths (the appended token included)
  int fused;          // 1: append the new token (position lens[s]) and attend over it
  int gblk;         // query heads handled together (matrix: G; vector: head block)
  int nhb;          // head blocks per KV head (matrix: 1)
  int ngroups;      // segments per sequence: g * nhb
  int slot_floats;  // gblk * d + round_up(2 * gblk, 4)
  int workgroups;   // persistent grid size P
  int seg_lead;     // empty schedule units ahead of each segment (piece start-up cost)
  int cnt_stride;   // ints between consecutive tickets
  int merge_kernel; // 1: shared segments are merged by merge_partials_kernel after this launch
  int merge_spread; // 1 (stream kernel): each part of a shared segment merges a slice of its heads at the end
  int* ws_stamp;    // spread merge: generation words and stamped flags (never reset)
  int2* seg_info;   // merge_kernel: per segment (p0, p1) of its shared pieces, p1 = -1 if none
  float scale_log2; // scale * log2(e)
  PagedLayout pg;   // paged caches (pg.table != nullptr); cap = table_stride << bs_log2
  int n_tok;        // query tokens per sequence (1: one-token decode; see head_row)
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The very end of the workspace: the fused step's completion counters (one
// top counter and 16 first-level ones, 128 bytes apart) in the first 4 KiB,
// then one ready flag per partial slot and folding wave of the stream kernel
// (kMaxWorkgroups x 2 slots x kFlagBlocks waves, int32).
constexpr size_t kFlagsOffset = 4096;
constexpr int kFlagBlocks = 2;
constexpr size_t kDoneBytes = kFlagsOffset + size_t(kMaxWorkgroups) * 2 * kFlagBlocks * sizeof(int);
// After those, the stamps of the spread merge (stream kernel): the launch
// generation and the generation whose workgroups have all started (first 256
// bytes), then one 64-bit flag per partial slot and folding wave holding the
// generation (low word) and a code (high word). They are never reset: a flag
// counts only when its generation is the current one (generations are
// nonzero, so zeroed flags never do), so the region is zero before the first
// call and then left as it is (or zeroed with the rest).
constexpr size_t kStampFlagsOffset = 256;
constexpr size_t kStampBytes = kStampFlagsOffset + size_t(kMaxWorkgroups) * 2 * kFlagBlocks * sizeof(uint64_t);

// y_s = x w_s^T for up to three weight matrices w_s [n_out_s][n_in] (bf16,
// packed by launch_pack_weight), x [rows][n_in], y_s [rows][n_out_s];
// blocks[s] = ceil(n_out_s / 16).
constexpr int kLinearMaxRows = 64;
struct LinearParams {
  const uint16_t* x;
  int rows, n_in, nseg;
  const uint16_t* w[3];
  uint16_t* y[3];
  int n_out[3];
  int blocks[3];
};

// dst[s][j][t][:] = mean of src[s][j*F + f][t][:] over f < F, t < rows_s
// (rows_s = min(lens[s], max_rows), or max_rows without lens); d % 8 == 0.
struct FoldParams {
  void* dst;
  const void* src;
  const int32_t* lens;
  int g_src, g_dst, cap_src, cap_dst, d, max_rows;
};

// Workspace layout, relative to the end of the caller's buffer so that a
// buffer sized for one shape serves every smaller shape without the regions
// of one call overlapping those of another: partial slots from the start,
// then (at the end) the tickets, kDoneBytes bytes of the fused step's
// counters and the slot flags, and the last kStampBytes bytes of spread-merge
// stamps. Tickets sit 128 bytes apart when b*h <= 8192, so that workgroups
// taking tickets of different segments at the same moment do not contend for
// one cache line; the ticket region never shrinks as b*h grows.
inline size_t counter_stride(int b, int h) { return size_t(b) * size_t(h) <= 8192 ? 32 : 1; }
inline size_t counter_ints(int b, int h) {
  const size_t bh = size_t(b) * size_t(h);
  return bh <= 8192 ? 32 * bh : (bh > 262144 ? bh : 262144);
}

struct WorkspaceLayout {
  size_t info_bytes, slot_bytes, cnt_bytes, total;
};

inline int slot_floats_for(int gblk, int d_v) { return gblk * d_v + ((2 * gblk + 3) & ~3); }

// gblk_bound: the largest head block any path may use for this shape;
// slot_wgs: the workgroups whose two partial slots are reserved (every
// possible grid: kMaxWorkgroups; a known grid: its size). From the start:
// the segment table of the separate merge (two ints per segment, at most
// b*h segments), then the partial slots; tickets at the end.
inline WorkspaceLayout workspace_layout(int b, int h, int gblk_bound, int d_v, int slot_wgs = kMaxWorkgroups) {
  WorkspaceLayout w;
  w.info_bytes = align256(size_t(b) * size_t(h) * 2 * sizeof(int));
  w.slot_bytes = align256(size_t(slot_wgs) * 2 * size_t(slot_floats_for(gblk_bound, d_v)) * sizeof(float));
  w.cnt_bytes = align256(counter_ints(b, h) * sizeof(int));
  w.total = w.info_bytes + w.slot_bytes + w.cnt_bytes + kDoneBytes + kStampBytes;
  return w;
}

// LDS the split merge needs (floats): (m, l) of kMergePairs (slot, head)
// pairs plus three per-head running values.
constexpr int kMergePairs = 8 * kMatrixMaxGroup;  // a batch of 8 slots for up to 64 heads
constexpr int kMergeLds = 2 * kMergePairs + 3 * kMatrixMaxGroup;

hipError_t launch_append(const AppendParams& p, int b, int dtype, hipStream_t stream);
hipError_t launch_decode_vector(const DecodeParams& p, int dtype, hipStream_t stream);
hipError_t launch_decode_matrix(const DecodeParams& p, hipStream_t stream);
// Matrix decode for up to 64 (virtual) heads per KV head and up to 64
// sequences (decode_stream.hip), one query token per sequence or a causal
// multi-token call; seg_lead counts empty tiles there.
constexpr int kStreamMaxGroup = 64;
constexpr int kStreamMaxBatch = 64;
hipError_t launch_decode_stream(const DecodeParams& p, hipStream_t stream);
int stream_workgroups_per_cu(bool fused, bool paged, int G);
hipError_t launch_merge_partials(const DecodeParams& p, int dtype, hipStream_t stream);
hipError_t launch_linear(const LinearParams& p, hipStream_t stream);
size_t packed_weight_bytes(int n_out, int n_in);
hipError_t launch_pack_weight(void* dst, const void* src, int n_out, int n_in, hipStream_t stream);
hipError_t launch_fold(const FoldParams& p, int b, int dtype, hipStream_t stream);
hipError_t launch_read_bandwidth(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t stream);

// Workgroups of the decode kernel instance that fit on one compute unit at
// once (runtime occupancy query, cached; 0 if the runtime cannot say).
int matrix_workgroups_per_cu(int G, bool fused, bool paged, bool causal = false);
// Waves per workgroup of the matrix kernel instance for G heads per KV head.
int matrix_waves(int G);
int vector_workgroups_per_cu(int dtype, int d, int heads_per_block, bool fused, bool paged, bool causal = false);
// The paged-cache and multi-token instances of the vector kernel (translation units of their own).
hipError_t launch_decode_vector_paged(const DecodeParams& p, int dtype, hipStream_t stream);
int vector_occupancy_paged(int dtype, int d, int heads_per_block, bool fused);
hipError_t launch_decode_vector_multi(const DecodeParams& p, int dtype, hipStream_t stream);
int vector_occupancy_multi(int dtype, int d, int heads_per_block);
hipError_t launch_decode_vector_multi_paged(const DecodeParams& p, int dtype, hipStream_t stream);
int vector_occupancy_multi_paged(int dtype, int d, int heads_per_block);
// Waves per workgroup of the vector kernel instance for this dtype, d and head block.
int vector_waves(int dtype, int d, int heads_per_block);

// Vector-path head block for G query heads per KV head: the smallest power of
// two >= G, capped at 8 (larger groups use several head blocks).
inline int vector_heads_per_block(int G) {
  if (G <= 1) return 1;
  if (G <= 2) return 2;
  if (G <= 4) return 4;
  return kVectorMaxBlock;
}

}  // namespace gqa

#if defined(__HIPCC__)
namespace gqa {

// ------------------------------------------------------------- addressing

// Row index (multiply by the head dim for elements) of position t of KV head
// j of sequence s: contiguous ((s*g + j)*cap + t), or, paged, row t mod B of
// head j in the block the table names for t (clamped into the pool, so a bad
// id reads or writes a wrong block of the pool, never outside it).
// UNIFORM: s and t are the same in every lane of the wave (the table entry is
// then read once, through the scalar unit).
template <bool PAGED, bool UNIFORM>
__device__ __forceinline__ size_t kv_row(const PagedLayout& pg, int g, int cap, int s, int j, int t) {
  if constexpr (PAGED) {
    int idx = s * pg.table_stride + (t >> pg.bs_log2);  // b * table_stride < 2^31 (host check)
    if constexpr (UNIFORM) idx = __builtin_amdgcn_readfirstlane(idx);
    const int blk = min(max(pg.table[idx], 0), pg.num_blocks - 1);
    return ((size_t(blk) * g + j) << pg.bs_log2) + (t & ((1 << pg.bs_log2) - 1));
  } else {
    return (size_t(s) * g + j) * size_t(cap) + t;
  }
}

// Multi-token decode: each KV group j serves GV = G * n_tok "virtual heads"
// v = r * G + i (token r, query head j*G + i), numbered V = j * GV + v over
// the sequence; q and out are [b][n_tok][h][d], so virtual head V of
// sequence s lives in row (s * n_tok + r) * h + j * G + i. With n_tok = 1
// that is row s * h + V. The one-token kernels instantiate the finishing
// code below with MULTI = false, where the row is s * h + V outright.
__device__ __forceinline__ size_t head_row(int n_tok, int h, int G, int s, int V) {
  if (n_tok == 1) return size_t(s) * h + V;
  const int GV = G * n_tok;
  const int j = V / GV, v = V - j * GV, r = v / G;
  return (size_t(s) * n_tok + r) * h + size_t(j) * G + (v - r * G);
}

// ---------------------------------------------------------------- numerics

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round fp32 to bf16 (nearest, ties to even); NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// 2^x on the hardware transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------- cross-lane reductions
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i within 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float xor_shuffle(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Sum over each aligned group of R consecutive lanes (R a power of two <= 64);
// every lane of the group receives the group sum.
template <int R>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (R >= 2) x += dpp<kDppQuadXor1>(x);
  if constexpr (R >= 4) x += dpp<kDppQuadXor2>(x);
  if constexpr (R >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (R >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (R >= 32) x += xor_shuffle(x, 16);
  if constexpr (R >= 64) x += xor_shuffle(x, 32);
  return x;
}

struct MergeWeights {
  float a, b;
};
// Weights that combine two split-softmax states with base-2 maxima m1, m2
// (either may be an empty state, m = -inf); m_out receives the joint max.
__device__ __forceinline__ MergeWeights merge_weights(float m1, float m2, float& m_out) {
  const float M = fmaxf(m1, m2);
  const float sub = (M == kNegInf) ? 0.0f : M;
  m_out = M;
  return {fast_exp2(m1 - sub), fast_exp2(m2 - sub)};
}

// ------------------------------------------------------- device-coherent I/O
// Buffer accesses with cache policy SC1 (device scope): stores write through
// to the device-coherent level and loads do not hit stale per-XCD copies.
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
constexpr int kCpolDevice = 16;                   // SC1
constexpr int kBufferWord3 = 0x00020000;          // raw (untyped) buffer resource

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slots_rsrc(const DecodeParams& p) {
  const int bytes = 2 * p.workgroups * p.slot_floats * int(sizeof(float));
  return __builtin_amdgcn_make_buffer_rsrc(p.ws_slots, 0, bytes, kBufferWord3);
}
__device__ __forceinline__ void coherent_store4(__amdgpu_buffer_rsrc_t r, int byte_off, f32x4v v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, v), r, byte_off, 0, kCpolDevice);
}
__device__ __forceinline__ void coherent_store1(__amdgpu_buffer_rsrc_t r, int byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, kCpolDevice);
}
__device__ __forceinline__ f32x4v coherent_load4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(f32x4v, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCpolDevice));
}
__device__ __forceinline__ float coherent_load1(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kCpolDevice));
}
// Wait until this wave's earlier memory writes have completed.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Effective attended length: lens clamped to [0, max_len]; for the fused step
// the stored length (before the append) is clamped to [0, max_len - 1] and
// the appended token adds one.
__device__ __forceinline__ int attended_len(const DecodeParams& p, int s) {
  int L = p.lens[s];
  L = L < 0 ? 0 : L;
  const int hi = p.max_len - p.fused;
  return (L > hi ? hi : L) + p.fused;
}

__device__ __forceinline__ int tiles_of(int L) { return sched::tiles_of(L); }
// Schedule units of a segment of length L (schedule.hpp). A unit is
// kUnitTiles tiles, one for each wave of a 4-wave workgroup, so that a piece
// made of whole units gives each of those waves the same number of tiles
// (only a segment's last unit can be short). The 8-wave matrix workgroups
// keep 4-tile units: 8-tile units, which would balance their waves the same
// way, measured slower (the coarser split of the work over workgroups costs
// more).
__device__ __forceinline__ int units_of(int L) { return sched::units_of<kUnitTiles>(L); }

// Units a non-empty segment occupies in the schedule: its units_of(L) real
// units preceded by p.seg_lead empty ones. The empty units carry no work;
// they stand for the cost of starting a piece (query load, wave merge,
// partial store and ticket), so that a workgroup whose range starts a new
// segment gets correspondingly fewer real units.
// LEAD = false: kernels launched with seg_lead = 0 compile the plain form.
template <bool LEAD>
__device__ __forceinline__ int sched_units_of(const DecodeParams& p, int L) {
  return int(sched::seg_units<kUnitTiles>(L, LEAD ? p.seg_lead : 0));
}

using sched::owner_of;
using sched::range_begin;

// Wave-level inclusive prefix sum over 64 lanes.
__device__ __forceinline__ long long wave_inclusive_scan(long long v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// Attended lengths as seen by one wave. For b <= 64 every lane keeps the
// length of sequence `lane` in a register after one load and lengths are
// read with a shuffle; larger batches read lens through the cache.
struct LensView {
  const DecodeParams* p;
  int reg;
  bool in_regs;
  __device__ void init(const DecodeParams& prm) {
    p = &prm;
    in_regs = prm.b <= 64;
    const int lane = threadIdx.x & 63;
    reg = (in_regs && lane < prm.b) ? attended_len(prm, lane) : 0;
  }
  // Length of sequence s (wave-uniform s, every lane active).
  __device__ int len(int s) const { return in_regs ? __shfl(reg, s, 64) : attended_len(*p, s); }
  // Length of sequence base + lane for the calling lane (0 beyond b).
  __device__ int lane_len(int base) const {
    const int s = base + (threadIdx.x & 63);
    if (in_regs) return base == 0 ? reg : 0;
    return s < p->b ? attended_len(*p, s) : 0;
  }
};

// Where the schedule puts the first unit of workgroup `workgroup`: the
// sequence s holding it (or b if the workgroup has no units), the unit index
// of that sequence's first unit, the total unit count T, and the number of
// workgroups that take part, P' = min(P, T), so that every taking part has a
// non-empty range. Every lane of the calling wave gets the same answer.
struct Located {
  long long total;
  long long seq_base;
  int s;
  int parts;
};
template <bool LEAD>
__device__ Located locate_units(const DecodeParams& p, const LensView& lv, int workgroup) {
  long long carry = 0;
  for (int base = 0; base < p.b; base += 64) {  // total units
    const long long v = (long long)p.ngroups * sched_units_of<LEAD>(p, lv.lane_len(base));
    const long long incl = wave_inclusive_scan(v);
    carry += __shfl(incl, 63, 64);
  }
  Located r;
  r.total = carry;
  r.parts = carry < p.workgroups ? int(carry) : p.workgroups;
  r.s = p.b;
  r.seq_base = carry;
  if (workgroup >= r.parts) return r;
  const long long u0 = range_begin(workgroup, carry, r.parts);
  carry = 0;
  for (int base = 0; base < p.b; base += 64) {
    const int s = base + (threadIdx.x & 63);
    const long long v = (long long)p.ngroups * sched_units_of<LEAD>(p, lv.lane_len(base));
    const long long incl = wave_inclusive_scan(v) + carry;
    const long long excl = incl - v;
    const unsigned long long hit = __ballot(s < p.b && v > 0 && excl <= u0 && u0 < incl);
    if (hit) {
      const int src = __ffsll((long long)hit) - 1;
      r.s = base + src;
      r.seq_base = __shfl(excl, src, 64);
      return r;
    }
    carry = __shfl(incl, 63, 64);
  }
  return r;
}

// One piece of a workgroup's range: tiles [tile_begin, tile_end) of segment
// (s, grp), i.e. positions [tile_begin*kTile, min(L, tile_end*kTile)).
// tile_begin is a multiple of the unit size. p0 and p1 are the first and last
// workgroups whose ranges touch the segment.
using Piece = sched::Piece;

// Iterates the pieces of workgroup `wg`'s unit range (schedule.hpp). LEAD:
// segments are preceded by p.seg_lead empty units.
template <bool LEAD>
struct PieceWalker {
  const DecodeParams* p;
  LensView lv;
  sched::Cursor c;

  __device__ void init(const DecodeParams& prm, int wg) {
    p = &prm;
    lv.init(prm);
    const Located loc = locate_units<LEAD>(prm, lv, wg);
    c.total = loc.total;
    c.parts = loc.parts;
    c.s = loc.s;
    c.seq_base = loc.seq_base;
    // A workgroup past the last taking part gets the empty range [0, 0).
    // Written as selects, not an early return: with two paths that each store
    // u and u_end, the compiler merges the stores through a pointer that picks
    // the field, which keeps both fields in scratch memory for the kernel's
    // whole life (a reload and a wait at every piece).
    const bool takes_part = wg < c.parts;
    const int parts_nz = c.parts > 0 ? c.parts : 1;
    c.u = takes_part ? range_begin(wg, c.total, parts_nz) : 0;
    c.u_end = takes_part ? range_begin(wg + 1, c.total, parts_nz) : 0;
  }

  __device__ bool more() const { return c.u < c.u_end; }

  __device__ bool next(Piece& pc) {
    const LensView& lens = lv;
    return sched::next_piece<kUnitTiles>([&lens](int s) { return lens.len(s); }, p->b, p->ngroups,
                                         LEAD ? p->seg_lead : 0, c, pc);
  }
};

// ------------------------------------------------------- piece finishing
template <typename TOut>
__device__ __forceinline__ void store_out(TOut* out, size_t idx, float v) {
  if constexpr (sizeof(TOut) == 2) out[idx] = f32_to_bf16(v);
  else out[idx] = v;
}

// A piece that shares its segment with other workgroups: the segment, its
// first and last workgroups, and the query heads [i0, i0 + nh) it covers.
struct SharedPiece {
  int s, grp, p0, p1, i0, nh;
  __device__ void set(const Piece& pc, int i0_, int nh_) {
    s = pc.s;
    grp = pc.grp;
    p0 = pc.p0;
    p1 = pc.p1;
    i0 = i0_;
    nh = nh_;
  }
};

__device__ __forceinline__ int* ticket_of(const DecodeParams& p, const SharedPiece& sh) {
  return p.ws_cnt + (size_t(sh.s) * p.ngroups + sh.grp) * p.cnt_stride;
}

// The combined state of a piece for query heads [i0, i0 + nh) sits in LDS:
// sm_m[nh], sm_l[nh] (base-2 max, sum) and sm_o[nh][d] (unnormalised output,
// 16-byte aligned). A segment inside one workgroup is written out directly by
// every thread.
template <bool MULTI>
__device__ __forceinline__ size_t out_row(const DecodeParams& p, int s, int V) {
  if constexpr (MULTI) return head_row(p.n_tok, p.h, p.G, s, V);
  else return size_t(s) * p.h + V;
}

template <typename TOut, bool MULTI>
__device__ void write_piece_out(const DecodeParams& p, int s, int i0, int nh, const float* sm_l,
                                const float* sm_o) {
  const int d = p.d;
  TOut* out = static_cast<TOut*>(p.out);
  if constexpr (MULTI) {
    for (int idx = threadIdx.x; idx < nh * d; idx += int(blockDim.x)) {
      const int hh = idx / d;
      const float l = sm_l[hh];
      store_out(out, out_row<true>(p, s, i0 + hh) * d + (idx - hh * d), l > 0.0f ? sm_o[idx] / l : 0.0f);
    }
  } else {
    const size_t out_row0 = (size_t(s) * p.h + i0) * d;
    for (int idx = threadIdx.x; idx < nh * d; idx += int(blockDim.x)) {
      const float l = sm_l[idx / d];
      store_out(out, out_row0 + idx, l > 0.0f ? sm_o[idx] / l : 0.0f);
    }
  }
}

// Store a shared piece's state into this workgroup's partial slot, with the
// threads tid, tid + nthr, ...: slot 1 if this workgroup owns the segment's
// first unit (the piece is the last of its range), slot 0 if not (the piece
// is the first of its range). The stores bypass the non-coherent caches.
__device__ void store_partial(const DecodeParams& p, const SharedPiece& sh, int wg, const float* sm_m,
                              const float* sm_l, const float* sm_o, int tid, int nthr) {
  const int d = p.d;
  const __amdgpu_buffer_rsrc_t rs = slots_rsrc(p);
  const int slot_bytes = p.slot_floats * int(sizeof(float));
  const int ml_off = p.gblk * d * int(sizeof(float));  // m then l after the o block
  const int mine = (wg * 2 + (wg == sh.p0 ? 1 : 0)) * slot_bytes;
  const int n4 = sh.nh * d / 4;
  for (int c4 = tid; c4 < n4; c4 += nthr)
    coherent_store4(rs, mine + c4 * 16, *reinterpret_cast<const f32x4v*>(sm_o + 4 * c4));
  for (int hh = tid; hh < sh.nh; hh += nthr) {
    coherent_store1(rs, mine + ml_off + hh * 4, sm_m[hh]);
    coherent_store1(rs, mine + ml_off + (p.gblk + hh) * 4, sm_l[hh]);
  }
}

// Merge of the n_slots partial states of one shared segment, by the
// workgroup that took its last ticket: slot 1 of p0 and slot 0 of
// p0+1 .. p1. Slots are read in batches of kMergeBatch; within a batch every
// (m, l) load and every partial-output load of this thread is issued before
// any is used, so a batch costs one memory round trip. Per-head running max,
// rescale factor and denominator live in LDS.
constexpr int kMergeBatch = 8;

template <typename TOut, int MAXC, bool MULTI>
__device__ void merge_segment(const DecodeParams& p, int s, int p0, int n_slots, int i0, int nh,
                              float* sm_merge) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int d = p.d;
  const __amdgpu_buffer_rsrc_t rs = slots_rsrc(p);
  const int slot_bytes = p.slot_floats * int(sizeof(float));
  const int ml_off = p.gblk * d * int(sizeof(float));
  const int n4 = nh * d / 4;
  float* pm = sm_merge;                // [kMergeBatch][nh] m, then weights
  float* pl = sm_merge + kMergePairs;  // [kMergeBatch][nh] l
  float* run_m = sm_merge + 2 * kMergePairs;
  float* run_den = run_m + kMatrixMaxGroup;
  float* run_r = run_den + kMatrixMaxGroup;
  f32x4v acc[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) acc[c] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
  for (int hh = tid; hh < nh; hh += nthr) {
    run_m[hh] = kNegInf;
    run_den[hh] = 0.0f;
  }
  for (int k0 = 0; k0 < n_slots; k0 += kMergeBatch) {
    const int kn = min(kMergeBatch, n_slots - k0);
    f32x4v o[kMergeBatch][MAXC];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const int kk = k0 + k;
      const int sb = ((p0 + kk) * 2 + (kk == 0 ? 1 : 0)) * slot_bytes;
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int c4 = tid + c * nthr;
        o[k][c] = (k < kn && c4 < n4) ? coherent_load4(rs, sb + c4 * 16) : f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
    for (int pair = tid; pair < kn * nh; pair += nthr) {
      const int k = pair / nh, hh = pair - k * nh;
      const int kk = k0 + k;
      const int sb = ((p0 + kk) * 2 + (kk == 0 ? 1 : 0)) * slot_bytes + ml_off;
      pm[pair] = coherent_load1(rs, sb + hh * 4);
      pl[pair] = coherent_load1(rs, sb + (p.gblk + hh) * 4);
    }
    __syncthreads();
    for (int hh = tid; hh < nh; hh += nthr) {
      float M = run_m[hh];
      for (int k = 0; k < kn; ++k) M = fmaxf(M, pm[k * nh + hh]);
      const float sub = (M == kNegInf) ? 0.0f : M;
      const float r = fast_exp2(run_m[hh] - sub);
      float den = run_den[hh] * r;
      for (int k = 0; k < kn; ++k) {
        const float wgt = fast_exp2(pm[k * nh + hh] - sub);
        den = fmaf(wgt, pl[k * nh + hh], den);
        pm[k * nh + hh] = wgt;
      }
      run_m[hh] = M;
      run_den[hh] = den;
      run_r[hh] = r;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int c4 = tid + c * nthr;
      if (c4 < n4) {
        const int hh = (4 * c4) / d;
        f32x4v a = acc[c] * run_r[hh];
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k)
          if (k < kn) a += pm[k * nh + hh] * o[k][c];
        acc[c] = a;
      }
    }
    // Every load of the batch has been used by now. The loads are issued and
    // used under the same condition, which the compiler's wait placement does
    // not pair up: without this compiler-visible wait it carries them as
    // outstanding past the merge and waits for all memory operations at the
    // top of the piece loop, i.e. for the stores of the previous piece, at
    // the start of every piece. (vmcnt(0); the other counters unconstrained.)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  TOut* out = static_cast<TOut*>(p.out);
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int c4 = tid + c * nthr;
    if (c4 < n4) {
      const int hh = (4 * c4) / d;
      const float den = run_den[hh];
      const float inv = den > 0.0f ? 1.0f / den : 0.0f;
      const size_t o0 = MULTI ? out_row<true>(p, s, i0 + hh) * d + (4 * c4 - hh * d)
                              : (size_t(s) * p.h + i0) * d + 4 * c4;
#pragma unroll
      for (int e = 0; e < 4; ++e) store_out(out, o0 + e, acc[c][e] * inv);
    }
  }
}

// Take the ticket of a shared piece whose partial every thread has just
// stored (after those stores have completed) and, if this workgroup arrived
// last, merge the segment and re-zero its ticket.
template <typename TOut, int MAXC, bool MULTI>
__device__ void settle_shared(const DecodeParams& p, const SharedPiece& sh, float* sm_merge, int* sm_flag) {
  wait_stores();
  __syncthreads();
  int* cnt = ticket_of(p, sh);
  if (threadIdx.x == 0) *sm_flag = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int n_slots = sh.p1 - sh.p0 + 1;
  const bool last = *sm_flag == n_slots - 1;
  __syncthreads();
  if (last) {
    merge_segment<TOut, MAXC, MULTI>(p, sh.s, sh.p0, n_slots, sh.i0, sh.nh, sm_merge);
    if (threadIdx.x == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The first piece of a range that more pieces follow, when it is shared.
// Settling it on the spot would stall the whole workgroup for a store
// acknowledgement and a ticket round trip while the memory system is busiest
// (measured at about 9 us). Instead wave 0 alone stores the partial (stored)
// and the other waves go straight on to the next piece; wave 0 waits for its
// stores and takes the ticket after its next tile (take), when they have
// long completed; the ticket's value is looked at once the range is done
// (resolve). The other workgroups of the segment hold it as their last or
// only piece, so this workgroup is rarely the last to arrive.
struct DeferredPiece {
  SharedPiece* sh;  // in LDS
  int state;        // 0 none, 1 partial stored, 2 ticket taken (wave 0's view)
  int ticket;       // lane 0 of wave 0
  __device__ void init(SharedPiece* lds) {
    sh = lds;
    state = 0;
  }
  // every thread; wave 0 stores
  __device__ void stored(const DecodeParams& p, const SharedPiece& piece, int wg, const float* sm_m,
                         const float* sm_l, const float* sm_o) {
    state = 1;
    if (threadIdx.x < 64) {
      if (threadIdx.x == 0) *sh = piece;
      store_partial(p, piece, wg, sm_m, sm_l, sm_o, threadIdx.x, 64);
    }
  }
  // wave 0 only, once per deferred piece
  __device__ void take(const DecodeParams& p) {
    wait_stores();
    if (threadIdx.x == 0)
      ticket = __hip_atomic_fetch_add(ticket_of(p, *sh), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    state = 2;
  }
  __device__ __forceinline__ void take_if_due(const DecodeParams& p, int wave) {
    if (wave == 0 && state == 1) take(p);
  }
  // every thread, after the range's last piece
  template <typename TOut, int MAXC, bool MULTI = false>
  __device__ void resolve(const DecodeParams& p, float* sm_merge, int* sm_flag) {
    if (state == 0) return;
    if (threadIdx.x < 64 && state == 1) take(p);
    __syncthreads();
    if (threadIdx.x == 0) *sm_flag = ticket;
    __syncthreads();
    const SharedPiece d = *sh;
    const int n_slots = d.p1 - d.p0 + 1;
    const bool last = *sm_flag == n_slots - 1;
    __syncthreads();
    if (last) {
      merge_segment<TOut, MAXC, MULTI>(p, d.s, d.p0, n_slots, d.i0, d.nh, sm_merge);
      if (threadIdx.x == 0) __hip_atomic_store(ticket_of(p, d), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
};

// Every thread, once the piece's combined state is in LDS: write it out,
// settle it, or defer it (see DeferredPiece).
template <typename TOut, int MAXC, bool MULTI = false>
__device__ void finish_piece(const DecodeParams& p, const Piece& pc, bool more_follow, int wg, int i0, int nh,
                             const float* sm_m, const float* sm_l, const float* sm_o, DeferredPiece& dfr,
                             float* sm_merge, int* sm_flag) {
  if (p.merge_kernel && pc.tile_begin == 0 && threadIdx.x == 0)
    p.seg_info[size_t(pc.s) * p.ngroups + pc.grp] = make_int2(pc.p0, pc.p0 == pc.p1 ? -1 : pc.p1);
  if (pc.p0 == pc.p1) {
    write_piece_out<TOut, MULTI>(p, pc.s, i0, nh, sm_l, sm_o);
    return;
  }
  SharedPiece sh;
  sh.set(pc, i0, nh);
  if (p.merge_kernel) {  // merged by the next launch: store and go on
    store_partial(p, sh, wg, sm_m, sm_l, sm_o, threadIdx.x, blockDim.x);
    return;
  }
  if (more_follow) {  // the first piece of the range (slot 0)
    dfr.stored(p, sh, wg, sm_m, sm_l, sm_o);
    return;
  }
  store_partial(p, sh, wg, sm_m, sm_l, sm_o, threadIdx.x, blockDim.x);
  settle_shared<TOut, MAXC, MULTI>(p, sh, sm_merge, sm_flag);
}

// Fused step: every workgroup counts itself out; the last one, which runs
// after every other workgroup has read lens for the last time, stores each
// sequence's new length and re-zeroes the counter.
__device__ void finish_step(const DecodeParams& p, int* sm_flag) {
  __syncthreads();
  if (threadIdx.x == 0)
    *sm_flag = __hip_atomic_fetch_add(p.ws_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (*sm_flag != int(gridDim.x) - 1) return;
  for (int s = threadIdx.x; s < p.b; s += int(blockDim.x)) p.lens[s] = attended_len(p, s);
  if (threadIdx.x == 0) __hip_atomic_store(p.ws_done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Zero the output rows of sequences that attend nothing; sequence s is
// handled by workgroup s mod P.
template <typename TOut, bool MULTI = false>
__device__ void zero_empty_sequences(const DecodeParams& p, int wg) {
  TOut* out = static_cast<TOut*>(p.out);
  for (int s = wg; s < p.b; s += p.workgroups) {
    if (attended_len(p, s) != 0) continue;
    if (p.merge_kernel)
      for (int k = threadIdx.x; k < p.ngroups; k += int(blockDim.x)) p.seg_info[size_t(s) * p.ngroups + k] = make_int2(0, -1);
    const int n_tok = MULTI ? p.n_tok : 1;
    const size_t row0 = size_t(s) * n_tok * p.h * p.d;  // the rows of all its tokens
    for (int idx = threadIdx.x; idx < n_tok * p.h * p.d; idx += int(blockDim.x)) out[row0 + idx] = TOut(0);
  }
}

}  // namespace gqa
#endif  // __HIPCC__
