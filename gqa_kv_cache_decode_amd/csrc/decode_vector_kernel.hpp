// Vector-ALU decode attention (every supported dtype and head dim).
//
// Computes, per sequence s and query head i with KV head j = floor(i / G),
//   out[s][i] = sum_t softmax_t(scale * q[s][i] . K[s][j][t]) V[s][j][t]
// (MQA review §2.1 Dot-Product Attention applied per head, with the cache of
// §2.4 / §3 and the contiguous head groups of the TF2 GQA lesson).
//
// A workgroup handles up to HB query heads of one group (a head block), so
// each K/V row fetched from HBM serves all of them. A K/V row is split over
// R = row_bytes / 16 consecutive lanes, each holding one 16-byte column; one
// wave load covers 64 / R consecutive rows (1 KiB, contiguous), and K/V are
// streamed with nontemporal loads. Dot products are summed across the R
// lanes with DPP row operations; every lane group keeps its own online-softmax
// state (base-2 running max, sum, unnormalised output), and the groups, then
// the waves (four or eight, through LDS), are merged at the end of each piece of the
// persistent schedule (gqa_internal.hpp), which finish_piece completes.
//
// The kernel template lives in this header so that its contiguous-cache
// instances (decode_vector.hip), paged-cache instances
// (decode_vector_paged.hip) and multi-token instances
// (decode_vector_multi.hip) compile as translation units of their own, in
// parallel.
#pragma once

#include "gqa_internal.hpp"

namespace gqa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ void widen16(const u32x4& r, float* f) {
  if constexpr (sizeof(T) == 4) {
    f[0] = __uint_as_float(r.x);
    f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z);
    f[3] = __uint_as_float(r.w);
  } else {
    f[0] = bf16_lo(r.x), f[1] = bf16_hi(r.x);
    f[2] = bf16_lo(r.y), f[3] = bf16_hi(r.y);
    f[4] = bf16_lo(r.z), f[5] = bf16_hi(r.z);
    f[6] = bf16_lo(r.w), f[7] = bf16_hi(r.w);
  }
}

template <typename T>
__device__ __forceinline__ u32x4 stream16(const T* ptr) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
}

template <typename T, int D, int HB>
struct Shape {
  static constexpr int VEC = 16 / int(sizeof(T));  // elements per 16-byte column
  static constexpr int R = D / VEC;                // lanes per row
  static_assert(R >= 1 && R <= 64 && (R & (R - 1)) == 0, "row must be 16..1024 bytes");
  static constexpr int RPW = 64 / R;                // rows per wave load
  static constexpr int NL = (kTile + RPW - 1) / RPW;  // loads per lane per tile
  static constexpr int UMAX = (HB >= 8 && VEC == 8) ? 2 : (HB >= 4 ? 4 : 8);
  static constexpr int U = NL < UMAX ? NL : UMAX;   // loads in flight per lane
  static constexpr int NSUB = NL / U;
  static_assert(NL % U == 0, "sub-batches must tile the 32-position tile");
  // Sub-batches unrolled in a tile: all of them, except with 256-dim rows
  // (one row per wave load, 32 sub-batches of loads), where unrolling lets
  // the compiler hoist later sub-batches' loads and run out of registers.
  static constexpr int SB_UNROLL = D >= 256 ? 1 : NSUB;
};

template <typename T, int D, int HB>
struct VState {
  static constexpr int VEC = Shape<T, D, HB>::VEC;
  float m[HB], l[HB], acc[HB][VEC];
};

// The appended token of a fused step: this lane's 16-byte column of its new
// rows and of its cache slot; `local` is its row within the current tile.
template <typename T>
struct NewRow {
  int local;
  const T* k;
  const T* v;
  T* kdst;
  T* vdst;
};

// One 32-position tile starting at row t0 (FULL: all rows valid). FUSED: the
// row nr.local is the appended token, read from its new rows and stored into
// the cache by the lanes that load it. CAUSAL (multi-token decode): head hh
// of the block only sees rows < lim[hh] (<= nvalid), its token's limit.
template <typename T, int D, int HB, bool FULL, bool FUSED, bool CAUSAL = false>
__device__ __forceinline__ void tile_step(VState<T, D, HB>& st, const float (&qf)[HB][Shape<T, D, HB>::VEC],
                                          const T* kbase, const T* vbase, int t0, int nvalid, int rg,
                                          const NewRow<T>& nr, const int* lim = nullptr) {
  using S = Shape<T, D, HB>;
  constexpr int VEC = S::VEC, U = S::U, RPW = S::RPW, R = S::R;
#pragma unroll S::SB_UNROLL
  for (int sb = 0; sb < S::NSUB; ++sb) {
    u32x4 kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = (sb * U + u) * RPW + rg;
      ok[u] = FULL ? (row < kTile) : (row < nvalid);
      if (FUSED && row == nr.local) {
        kr[u] = *reinterpret_cast<const u32x4*>(nr.k);
        vr[u] = *reinterpret_cast<const u32x4*>(nr.v);
        *reinterpret_cast<u32x4*>(nr.kdst) = kr[u];
        *reinterpret_cast<u32x4*>(nr.vdst) = vr[u];
      } else if (ok[u]) {
        kr[u] = stream16(kbase + size_t(t0 + row) * D);
        vr[u] = stream16(vbase + size_t(t0 + row) * D);
      } else {
        kr[u] = u32x4{0u, 0u, 0u, 0u};
        vr[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    float sc[U][HB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[VEC];
      widen16<T>(kr[u], kf);
#pragma unroll
      for (int hh = 0; hh < HB; ++hh) {
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) part = fmaf(qf[hh][e], kf[e], part);
        part = group_sum<R>(part);
        if constexpr (CAUSAL) sc[u][hh] = (ok[u] && (sb * U + u) * RPW + rg < lim[hh]) ? part : kNegInf;
        else sc[u][hh] = ok[u] ? part : kNegInf;
      }
    }
    float vf[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) widen16<T>(vr[u], vf[u]);
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      float mx = sc[0][hh];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u][hh]);
      const float mn = fmaxf(st.m[hh], mx);
      const float sub = (mn == kNegInf) ? 0.0f : mn;
      const float alpha = fast_exp2(st.m[hh] - sub);
      st.m[hh] = mn;
      float pu[U];
      float psum = 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        pu[u] = fast_exp2(sc[u][hh] - sub);
        psum += pu[u];
      }
      st.l[hh] = fmaf(st.l[hh], alpha, psum);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float a = st.acc[hh][e] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) a = fmaf(pu[u], vf[u][e], a);
        st.acc[hh][e] = a;
      }
    }
  }
}

// Waves per workgroup: eight (one workgroup per compute unit) when a head
// block's accumulators are small enough for two waves per SIMD, else four.
template <typename T, int D, int HB>
constexpr int vector_waves_of() {
  return (HB <= 4 && HB * D * int(sizeof(T)) <= 512) ? 8 : 4;
}

// PAGED: K/V live in block pools addressed through the block table (one
// lookup per 32-position tile); otherwise in contiguous [b][g][cap][d] caches.
// CAUSAL: multi-token decode; each KV group has GV = G * n_tok virtual heads
// (token r, head i; see head_row), taken HB at a time, and token r's heads
// see positions < L - (n_tok - 1 - r).
template <typename T, int D, int HB, bool FUSED, bool PAGED, bool CAUSAL = false>
__global__ __launch_bounds__((vector_waves_of<T, D, HB>() * 64)) void decode_vector_kernel(DecodeParams p) {
  constexpr int WAVES = vector_waves_of<T, D, HB>();
  constexpr int THREADS = WAVES * 64;
  constexpr int MAXC = (HB * D / 4 + THREADS - 1) / THREADS;
  using S = Shape<T, D, HB>;
  constexpr int VEC = S::VEC, R = S::R;

  __shared__ float sm_m[WAVES][HB];
  __shared__ float sm_l[WAVES][HB];
  __shared__ float sm_o[WAVES][HB][D];
  __shared__ float fin_m[HB];
  __shared__ float fin_l[HB];
  __shared__ __attribute__((aligned(16))) float fin_o[HB][D];
  __shared__ float sm_merge[kMergeLds];
  __shared__ int s_flag;
  __shared__ SharedPiece s_deferred;

  const int wg = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int col = lane % R;
  const int rg = lane / R;

  zero_empty_sequences<T, CAUSAL>(p, wg);
  const int GV = CAUSAL ? p.G * p.n_tok : p.G;  // (virtual) heads per KV group

  PieceWalker<false> walker;
  walker.init(p, wg);
  Piece pc;
  DeferredPiece dfr;
  dfr.init(&s_deferred);
  while (walker.next(pc)) {
    const int s = pc.s;
    const int j = pc.grp / p.nhb;
    const int hb = pc.grp - j * p.nhb;
    const int i0 = j * GV + hb * HB;
    const int nh = min(HB, GV - hb * HB);

    // query rows of the head block, widened and pre-multiplied by scale*log2(e)
    float qf[HB][VEC];
    const T* qrow = static_cast<const T*>(p.q) + (size_t(s) * p.h + i0) * D + col * VEC;
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      if (hh < nh) {
        const T* qp = CAUSAL ? static_cast<const T*>(p.q) + head_row(p.n_tok, p.h, p.G, s, i0 + hh) * D + col * VEC
                             : qrow + size_t(hh) * D;
        const u32x4 raw = *reinterpret_cast<const u32x4*>(qp);
        widen16<T>(raw, qf[hh]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) qf[hh][e] *= p.scale_log2;
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) qf[hh][e] = 0.0f;
      }
    }
    VState<T, D, HB> st;
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      st.m[hh] = kNegInf;
      st.l[hh] = 0.0f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) st.acc[hh][e] = 0.0f;
    }
    const size_t kv_head = size_t(s) * p.g + j;
    const T* kbase = static_cast<const T*>(p.k_cache) + kv_head * p.cap * D + col * VEC;
    const T* vbase = static_cast<const T*>(p.v_cache) + kv_head * p.cap * D + col * VEC;
    const int t_end = min(pc.L, pc.tile_end * kTile);
    const int pos_new = FUSED ? pc.L - 1 : -1;  // the appended token (fused step)
    // CAUSAL: how many of the last positions head hh does not see
    int hide[HB];
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) hide[hh] = (CAUSAL && hh < nh) ? p.n_tok - 1 - (hb * HB + hh) / p.G : 0;
    const int hide_max = CAUSAL ? p.n_tok - 1 : 0;
    for (int tile = pc.tile_begin + w; tile < pc.tile_end; tile += WAVES) {
      const int t0 = tile * kTile;
      const int nvalid = t_end - t0;
      // rows of this tile: kb/vb + (tb + r) * D, r < 32 (this lane's column included)
      const T* kb = kbase;
      const T* vb = vbase;
      int tb = t0;
      if constexpr (PAGED) {
        const size_t row = kv_row<true, true>(p.pg, p.g, p.cap, s, j, t0);
        kb = static_cast<const T*>(p.k_cache) + row * D + col * VEC;
        vb = static_cast<const T*>(p.v_cache) + row * D + col * VEC;
        tb = 0;
      }
      if (FUSED && pos_new >= t0 && pos_new < t0 + kTile) {
        // the segment's last tile: take the new row from k_new / v_new and store it
        NewRow<T> nr;
        nr.local = pos_new - t0;
        nr.k = static_cast<const T*>(p.k_new) + kv_head * D + col * VEC;
        nr.v = static_cast<const T*>(p.v_new) + kv_head * D + col * VEC;
        const size_t new_row = kv_row<PAGED, true>(p.pg, p.g, p.cap, s, j, pos_new);
        nr.kdst = static_cast<T*>(p.k_cache) + new_row * D + col * VEC;
        nr.vdst = static_cast<T*>(p.v_cache) + new_row * D + col * VEC;
        tile_step<T, D, HB, false, true>(st, qf, kb, vb, tb, nvalid, rg, nr);
      } else if (nvalid >= kTile && (!CAUSAL || pc.L - t0 - hide_max >= kTile)) {
        tile_step<T, D, HB, true, false>(st, qf, kb, vb, tb, kTile, rg, NewRow<T>{});
      } else if constexpr (CAUSAL) {
        int lim[HB];
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) lim[hh] = min(nvalid, pc.L - t0 - hide[hh]);
        tile_step<T, D, HB, false, false, true>(st, qf, kb, vb, tb, nvalid, rg, NewRow<T>{}, lim);
      } else {
        tile_step<T, D, HB, false, false>(st, qf, kb, vb, tb, nvalid, rg, NewRow<T>{});
      }
      dfr.take_if_due(p, w);
    }

    // merge the lane groups of the wave (same column, different rows)
#pragma unroll
    for (int off = R; off < 64; off <<= 1) {
#pragma unroll
      for (int hh = 0; hh < HB; ++hh) {
        const float mo = xor_shuffle(st.m[hh], off);
        const float lo = xor_shuffle(st.l[hh], off);
        float mn;
        const MergeWeights wt = merge_weights(st.m[hh], mo, mn);
        st.l[hh] = st.l[hh] * wt.a + lo * wt.b;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float ao = xor_shuffle(st.acc[hh][e], off);
          st.acc[hh][e] = st.acc[hh][e] * wt.a + ao * wt.b;
        }
        st.m[hh] = mn;
      }
    }
    if (rg == 0) {
#pragma unroll
      for (int hh = 0; hh < HB; ++hh) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) sm_o[w][hh][col * VEC + e] = st.acc[hh][e];
        if (col == 0) {
          sm_m[w][hh] = st.m[hh];
          sm_l[w][hh] = st.l[hh];
        }
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < HB * D; idx += THREADS) {
      const int hh = idx / D, dd = idx - hh * D;
      float M = sm_m[0][hh];
#pragma unroll
      for (int ww = 1; ww < WAVES; ++ww) M = fmaxf(M, sm_m[ww][hh]);
      const float sub = (M == kNegInf) ? 0.0f : M;
      float o = 0.0f, lsum = 0.0f;
#pragma unroll
      for (int ww = 0; ww < WAVES; ++ww) {
        const float wgt = fast_exp2(sm_m[ww][hh] - sub);
        o = fmaf(wgt, sm_o[ww][hh][dd], o);
        lsum = fmaf(wgt, sm_l[ww][hh], lsum);
      }
      fin_o[hh][dd] = o;
      if (dd == 0) {
        fin_m[hh] = M;
        fin_l[hh] = lsum;
      }
    }
    __syncthreads();
    finish_piece<T, MAXC, CAUSAL>(p, pc, walker.more(), wg, i0, nh, fin_m, fin_l, &fin_o[0][0], dfr, sm_merge,
                                 &s_flag);
  }
  dfr.resolve<T, MAXC, CAUSAL>(p, sm_merge, &s_flag);
  if (FUSED) finish_step(p, &s_flag);
}

// CAUSAL instances exist without FUSED (the multi-token append is its own launch).
template <typename T, int D, int HB, bool PAGED, bool CAUSAL>
hipError_t launch_one(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid(p.workgroups), block(vector_waves_of<T, D, HB>() * 64);
  if constexpr (CAUSAL)
    hipLaunchKernelGGL((decode_vector_kernel<T, D, HB, false, PAGED, true>), grid, block, 0, stream, p);
  else if (p.fused)
    hipLaunchKernelGGL((decode_vector_kernel<T, D, HB, true, PAGED>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((decode_vector_kernel<T, D, HB, false, PAGED>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D, bool PAGED, bool CAUSAL>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  switch (p.gblk) {
    case 1: return launch_one<T, D, 1, PAGED, CAUSAL>(p, stream);
    case 2: return launch_one<T, D, 2, PAGED, CAUSAL>(p, stream);
    case 4: return launch_one<T, D, 4, PAGED, CAUSAL>(p, stream);
    default: return launch_one<T, D, 8, PAGED, CAUSAL>(p, stream);
  }
}

template <typename T, bool PAGED, bool CAUSAL>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  switch (p.d) {
    case 16: return launch_d<T, 16, PAGED, CAUSAL>(p, stream);
    case 32: return launch_d<T, 32, PAGED, CAUSAL>(p, stream);
    case 64: return launch_d<T, 64, PAGED, CAUSAL>(p, stream);
    case 128: return launch_d<T, 128, PAGED, CAUSAL>(p, stream);
    case 256: return launch_d<T, 256, PAGED, CAUSAL>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool PAGED, bool CAUSAL = false>
hipError_t launch_vector(const DecodeParams& p, int dtype, hipStream_t stream) {
  return dtype == 0 ? launch_t<float, PAGED, CAUSAL>(p, stream) : launch_t<uint16_t, PAGED, CAUSAL>(p, stream);
}


template <typename T, int D, bool FUSED, bool PAGED, bool CAUSAL>
int occupancy_d(int hb) {
  int n = 0;
  hipError_t e;
  switch (hb) {
    case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_vector_kernel<T, D, 1, FUSED, PAGED, CAUSAL>, vector_waves_of<T, D, 1>() * 64, 0); break;
    case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_vector_kernel<T, D, 2, FUSED, PAGED, CAUSAL>, vector_waves_of<T, D, 2>() * 64, 0); break;
    case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_vector_kernel<T, D, 4, FUSED, PAGED, CAUSAL>, vector_waves_of<T, D, 4>() * 64, 0); break;
    default: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_vector_kernel<T, D, 8, FUSED, PAGED, CAUSAL>, vector_waves_of<T, D, 8>() * 64, 0); break;
  }
  if (e != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

template <typename T, bool FUSED, bool PAGED, bool CAUSAL>
int occupancy_t(int d, int hb) {
  switch (d) {
    case 16: return occupancy_d<T, 16, FUSED, PAGED, CAUSAL>(hb);
    case 32: return occupancy_d<T, 32, FUSED, PAGED, CAUSAL>(hb);
    case 64: return occupancy_d<T, 64, FUSED, PAGED, CAUSAL>(hb);
    case 128: return occupancy_d<T, 128, FUSED, PAGED, CAUSAL>(hb);
    default: return occupancy_d<T, 256, FUSED, PAGED, CAUSAL>(hb);
  }
}

// Workgroups of one instance that fit on a compute unit (0 if unknown).
template <bool PAGED, bool CAUSAL = false>
int vector_occupancy(int dtype, int d, int hb, bool fused) {
  if constexpr (CAUSAL) {
    return dtype == 0 ? occupancy_t<float, false, PAGED, true>(d, hb) : occupancy_t<uint16_t, false, PAGED, true>(d, hb);
  } else {
    if (fused)
      return dtype == 0 ? occupancy_t<float, true, PAGED, false>(d, hb) : occupancy_t<uint16_t, true, PAGED, false>(d, hb);
    return dtype == 0 ? occupancy_t<float, false, PAGED, false>(d, hb) : occupancy_t<uint16_t, false, PAGED, false>(d, hb);
  }
}


}  // namespace
}  // namespace gqa
