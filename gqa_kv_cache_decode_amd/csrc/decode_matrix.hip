// Matrix-core (MFMA) decode attention: bf16 K/V/q, d_k = d_v = 128, fp32
// accumulation, up to 64 query heads per KV head.
//
// Same result as the vector path (MQA review §2.1 per query head over the
// cache of §2.4 / §3; contiguous head groups of the TF2 GQA lesson). Both
// contractions of a G-head group against a 32-position tile are small dense
// matrix products, so they run on v_mfma_f32_16x16x32_bf16 with the G query
// heads padded to 16 (NB blocks of 16 heads):
//
//   scores  S^T[t][i] = sum_k K[t][k] * Q^T[k][i]   A = K tile, B = Q^T
//   output  O^T[v][i] += sum_t V^T[v][t] * P^T[t][i] A = V^T tile, B = P^T
//
// Operand layout of the 16x16x32 MFMA (A: 16 rows x 32 k, B: 32 k x 16
// columns, C: 16 x 16): lane l supplies row / column (l % 16) and the 8
// k-slots of group (l / 16); lane l receives C rows 4*(l/16) .. +3 of column
// l % 16. The contraction only needs A and B to agree on which k each
// (group, slot) stands for, which is how the kernel picks K dims and V
// positions freely:
//
// * K: lane (n = l%16, q = l/16) loads 16 bytes of row 16*sg + n (sg =
//   sub-tile 0/1) at dims 32*ks + 8*q, ks = 0..3: exactly the A operand.
// * The score MFMA leaves lane (n, q) with positions 16*sg + 4q + 0..3 of
//   head n: these 8 probabilities, packed to bf16, are the B operand of the
//   value MFMA for k-group q, with k-slot r <-> position tau(q, r) =
//   4q + r (r < 4) or 16 + 4q + (r - 4).
// * V: lane (n, q) loads 16 bytes (dims 8n .. 8n+7) of the 8 rows tau(q, r);
//   a quarter-wave reads whole 256-byte rows. An 8 x 8 transpose of 16-bit
//   values inside the lane gives, for each e = 0..7, the 8 positions of dim
//   8n + e: the A operand of value MFMA e, whose output row m is dim 8m + e.
//   Lane (n, q) therefore accumulates dims 32q .. 32q + 31 of head n.
//
// K and V are streamed once with nontemporal loads (they are not reused, and
// keeping them out of the caches measurably raises HBM read bandwidth).
// Workgroups follow the persistent schedule of gqa_internal.hpp; inside a
// piece each wave walks every WAVES-th tile with an online softmax (base 2,
// running max per head shared by the 4 lanes of a head), and the waves are
// merged through LDS before the piece is published.
//
// FUSED (the decode step): the tile holding the appended token takes that
// row from k_new / v_new instead of the cache and writes it to its cache
// slot; the last workgroup to finish stores the grown lengths.
#include <atomic>

#include "gqa_internal.hpp"

namespace gqa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr int OPAD = 4;  // LDS row padding (floats) against bank conflicts
constexpr int kMatrixWaves1 = 8;  // waves per workgroup of the one-head-block kernel

__device__ __forceinline__ u32x4 load16(const uint16_t* ptr) {
  return *reinterpret_cast<const u32x4*>(ptr);
}
__device__ __forceinline__ u32x4 stream16(const uint16_t* ptr) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ int v_row(int q4, int r) { return (r < 4) ? (4 * q4 + r) : (16 + 4 * q4 + (r - 4)); }

// Value-MFMA A operand e from the 8 loaded V rows (vr[r] holds dims 8n..8n+7
// of position tau(q, r)): dword k = (dim 8n+e of row 2k, of row 2k+1).
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

// The appended token of a fused step: its rows in k_new / v_new and its cache
// slot. `local` is its row within the current tile (outside [0, 32): none).
struct NewRow {
  int local;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* kdst;
  uint16_t* vdst;
};

__device__ __forceinline__ void store16(uint16_t* ptr, u32x4 v) { *reinterpret_cast<u32x4*>(ptr) = v; }

template <int NB>
struct WaveState {
  f32x4 oacc[NB][8];
  float mrun[NB], lrun[NB];
};

// One 32-position tile starting at kbase/vbase row t0 (FULL: all 32 rows
// valid; otherwise only rows < nvalid are read). FUSED: the row nr.local is
// the appended token, read from its new rows and stored into the cache by the
// lanes that load it. CAUSAL (multi-token decode): this lane's head column of
// block nb only sees rows < lim[nb] (<= nvalid), its token's causal limit.
template <int NB, bool FULL, bool FUSED, bool CAUSAL = false>
__device__ __forceinline__ void tile_step(WaveState<NB>& st, const bf16x8 (&qop)[NB][4], const uint16_t* kbase,
                                          const uint16_t* vbase, int t0, int nvalid, float sl2, int n16,
                                          int q4, const NewRow& nr, const int* lim = nullptr) {
  u32x4 kr[2][4];
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {
    const int row = 16 * sg + n16;
    const uint16_t* kp = kbase + size_t(t0 + row) * D + q4 * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (FUSED && row == nr.local) {
        kr[sg][ks] = load16(nr.k + q4 * 8 + ks * 32);
        store16(nr.kdst + q4 * 8 + ks * 32, kr[sg][ks]);
      } else if (FULL || row < nvalid) {
        kr[sg][ks] = stream16(kp + ks * 32);
      } else {
        kr[sg][ks] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  u32x4 vr[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int row = v_row(q4, r);
    if (FUSED && row == nr.local) {
      vr[r] = load16(nr.v + n16 * 8);
      store16(nr.vdst + n16 * 8, vr[r]);
    } else if (FULL || row < nvalid) {
      vr[r] = stream16(vbase + size_t(t0 + row) * D + n16 * 8);
    } else {
      vr[r] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  bf16x8 pop[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float sv[8];
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
      f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[sg][ks]), qop[nb][ks], sacc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * sg + 4 * q4 + i;
        if constexpr (CAUSAL) sv[sg * 4 + i] = (FULL || row < lim[nb]) ? sacc[i] * sl2 : kNegInf;
        else sv[sg * 4 + i] = (FULL || row < nvalid) ? sacc[i] * sl2 : kNegInf;
      }
    }
    float mx = sv[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) mx = fmaxf(mx, sv[k]);
    mx = fmaxf(mx, xor_shuffle(mx, 16));
    mx = fmaxf(mx, xor_shuffle(mx, 32));
    const float mn = fmaxf(st.mrun[nb], mx);
    const float sub = (mn == kNegInf) ? 0.0f : mn;
    const float alpha = fast_exp2(st.mrun[nb] - sub);
    st.mrun[nb] = mn;
    float psum = 0.0f;
    bf16x8 pk;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const __bf16 pb = static_cast<__bf16>(fast_exp2(sv[k] - sub));
      pk[k] = pb;
      psum += static_cast<float>(pb);  // the denominator sums the weights actually applied
    }
    pop[nb] = pk;
    st.lrun[nb] = fmaf(st.lrun[nb], alpha, psum);
#pragma unroll
    for (int e = 0; e < 8; ++e) st.oacc[nb][e] *= alpha;
  }
#define GQA_PV_STEP(E)                                                                           \
  {                                                                                              \
    const bf16x8 va = v_transpose<E>(vr);                                                        \
    _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) st.oacc[nb][E] =                           \
        __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop[nb], st.oacc[nb][E], 0, 0, 0);           \
  }
  GQA_PV_STEP(0) GQA_PV_STEP(1) GQA_PV_STEP(2) GQA_PV_STEP(3)
  GQA_PV_STEP(4) GQA_PV_STEP(5) GQA_PV_STEP(6) GQA_PV_STEP(7)
#undef GQA_PV_STEP
}

// WAVES = 8 (one head block): one 512-thread workgroup per compute unit. Two
// 4-wave workgroups per unit were measured slower: the one dispatched second
// streams about a tenth slower than its partner (older waves win the issue
// arbitration) and the unit's work ends with it, while the eight waves of one
// workgroup share each piece and meet at its barriers. WAVES = 4: the larger
// head blocks, whose register needs allow one 4-wave workgroup per unit.
// PAGED: K/V live in block pools addressed through the block table (one
// lookup per 32-position tile); otherwise in contiguous [b][g][cap][d] caches.
// CAUSAL: multi-token decode; the group's heads are the GV = G * n_tok
// virtual heads (token r, head i) of head_row, every K/V tile is read once
// for all of them, and token r's heads see positions < L - (n_tok - 1 - r).
template <int NB, bool FUSED, int WAVES, bool PAGED, bool CAUSAL>
__global__ __launch_bounds__(WAVES * 64, (NB == 1 && WAVES == 4) ? 2 : 1) void decode_matrix_kernel(DecodeParams p) {
  constexpr int THREADS = WAVES * 64;
  __shared__ float sm_m[WAVES][16];
  __shared__ float sm_l[WAVES][16];
  __shared__ __attribute__((aligned(16))) float sm_o[WAVES][16][D + OPAD];
  __shared__ float fin_m[NB * 16];
  __shared__ float fin_l[NB * 16];
  __shared__ __attribute__((aligned(16))) float fin_o[NB * 16][D];
  __shared__ float sm_merge[kMergeLds];
  __shared__ int s_flag;
  __shared__ SharedPiece s_deferred;

  const int wg = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n16 = lane & 15;
  const int q4 = lane >> 4;
  const int G = CAUSAL ? p.G * p.n_tok : p.G;  // (virtual) heads per KV group
  const float sl2 = p.scale_log2;

  zero_empty_sequences<uint16_t, CAUSAL>(p, wg);

  PieceWalker<true> walker;
  walker.init(p, wg);
  Piece pc;
  DeferredPiece dfr;
  dfr.init(&s_deferred);
  while (walker.next(pc)) {
    const int s = pc.s, j = pc.grp;
    const int i0 = j * G;
    // Q^T operands: head nb*16 + n16, dims 32*ks + 8*q4 .. +7 (zero for padding heads).
    bf16x8 qop[NB][4];
    const uint16_t* qg = static_cast<const uint16_t*>(p.q) + (size_t(s) * p.h + i0) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int head = nb * 16 + n16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if constexpr (CAUSAL) {
          if (head < G)
            v = load16(static_cast<const uint16_t*>(p.q) + head_row(p.n_tok, p.h, p.G, s, i0 + head) * D + ks * 32 +
                       q4 * 8);
        } else {
          if (head < G) v = load16(qg + size_t(head) * D + ks * 32 + q4 * 8);
        }
        qop[nb][ks] = as_bf16x8(v);
      }
    }
    WaveState<NB> st;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      st.mrun[nb] = kNegInf;
      st.lrun[nb] = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.oacc[nb][e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const size_t kv_head = size_t(s) * p.g + j;
    const uint16_t* kbase = static_cast<const uint16_t*>(p.k_cache) + kv_head * p.cap * D;
    const uint16_t* vbase = static_cast<const uint16_t*>(p.v_cache) + kv_head * p.cap * D;
    const int t_end = min(pc.L, pc.tile_end * kTile);
    const int pos_new = FUSED ? pc.L - 1 : -1;  // the appended token (fused step)
    // CAUSAL: how many of the last positions this lane's head column does not
    // see (n_tok - 1 - its token); padding columns see what the last token sees
    int hide[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int head = nb * 16 + n16;
      hide[nb] = (CAUSAL && head < G) ? p.n_tok - 1 - head / p.G : 0;
    }
    const int hide_max = CAUSAL ? p.n_tok - 1 : 0;
    for (int tile = pc.tile_begin + w; tile < pc.tile_end; tile += WAVES) {
      const int t0 = tile * kTile;
      const int nvalid = t_end - t0;
      // rows of this tile: kb/vb + (tb + r) * D, r < 32
      const uint16_t* kb = kbase;
      const uint16_t* vb = vbase;
      int tb = t0;
      if constexpr (PAGED) {
        const size_t row = kv_row<true, true>(p.pg, p.g, p.cap, s, j, t0);
        kb = static_cast<const uint16_t*>(p.k_cache) + row * D;
        vb = static_cast<const uint16_t*>(p.v_cache) + row * D;
        tb = 0;
      }
      if (FUSED && pos_new >= t0 && pos_new < t0 + kTile) {
        // the segment's last tile: take the new row from k_new / v_new and store it
        NewRow nr;
        nr.local = pos_new - t0;
        nr.k = static_cast<const uint16_t*>(p.k_new) + kv_head * D;
        nr.v = static_cast<const uint16_t*>(p.v_new) + kv_head * D;
        const size_t new_row = kv_row<PAGED, true>(p.pg, p.g, p.cap, s, j, pos_new);
        nr.kdst = static_cast<uint16_t*>(p.k_cache) + new_row * D;
        nr.vdst = static_cast<uint16_t*>(p.v_cache) + new_row * D;
        tile_step<NB, false, true>(st, qop, kb, vb, tb, nvalid, sl2, n16, q4, nr);
      } else if (nvalid >= kTile && (!CAUSAL || pc.L - t0 - hide_max >= kTile)) {
        tile_step<NB, true, false>(st, qop, kb, vb, tb, kTile, sl2, n16, q4, NewRow{});
      } else if constexpr (CAUSAL) {
        int lim[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) lim[nb] = min(nvalid, pc.L - t0 - hide[nb]);
        tile_step<NB, false, false, true>(st, qop, kb, vb, tb, nvalid, sl2, n16, q4, NewRow{}, lim);
      } else {
        tile_step<NB, false, false>(st, qop, kb, vb, tb, nvalid, sl2, n16, q4, NewRow{});
      }
      dfr.take_if_due(p, w);
    }

    // merge the waves through LDS, one 16-head block at a time
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float lsum = st.lrun[nb];
      lsum += xor_shuffle(lsum, 16);
      lsum += xor_shuffle(lsum, 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // dims 32*q4 + 8*i + e, e = 0..7
        f32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = st.oacc[nb][e][i];
          hi[e] = st.oacc[nb][e + 4][i];
        }
        *reinterpret_cast<f32x4*>(&sm_o[w][n16][32 * q4 + 8 * i]) = lo;
        *reinterpret_cast<f32x4*>(&sm_o[w][n16][32 * q4 + 8 * i + 4]) = hi;
      }
      if (q4 == 0) {
        sm_m[w][n16] = st.mrun[nb];
        sm_l[w][n16] = lsum;
      }
      __syncthreads();
      const int nh_blk = min(16, G - nb * 16);
      // one 16-byte column of one head per thread: the head's weights are
      // computed once for its four outputs
      constexpr int C4 = D / 4;
      for (int idx = threadIdx.x; idx < nh_blk * C4; idx += THREADS) {
        const int hh = idx / C4, c4 = idx - hh * C4;
        float M = sm_m[0][hh];
#pragma unroll
        for (int ww = 1; ww < WAVES; ++ww) M = fmaxf(M, sm_m[ww][hh]);
        const float sub = (M == kNegInf) ? 0.0f : M;
        f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
        float ls = 0.0f;
#pragma unroll
        for (int ww = 0; ww < WAVES; ++ww) {
          const float wgt = fast_exp2(sm_m[ww][hh] - sub);
          const f32x4 ov = *reinterpret_cast<const f32x4*>(&sm_o[ww][hh][4 * c4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = fmaf(wgt, ov[e], o[e]);
          ls = fmaf(wgt, sm_l[ww][hh], ls);
        }
        *reinterpret_cast<f32x4*>(&fin_o[nb * 16 + hh][4 * c4]) = o;
        if (c4 == 0) {
          fin_m[nb * 16 + hh] = M;
          fin_l[nb * 16 + hh] = ls;
        }
      }
      __syncthreads();
    }
    finish_piece<uint16_t, NB * 8 / WAVES, CAUSAL>(p, pc, walker.more(), wg, i0, G, fin_m, fin_l, &fin_o[0][0], dfr,
                                           sm_merge, &s_flag);
  }
  dfr.resolve<uint16_t, NB * 8 / WAVES, CAUSAL>(p, sm_merge, &s_flag);
  if (FUSED) finish_step(p, &s_flag);
}

template <bool FUSED, bool PAGED, bool CAUSAL>
void launch_nb(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid(p.workgroups);
  const int GV = p.G * p.n_tok;
  if (GV <= 16) {
    hipLaunchKernelGGL((decode_matrix_kernel<1, FUSED, kMatrixWaves1, PAGED, CAUSAL>), grid,
                       dim3(kMatrixWaves1 * 64), 0, stream, p);
  } else if (GV <= 32) {
    hipLaunchKernelGGL((decode_matrix_kernel<2, FUSED, 4, PAGED, CAUSAL>), grid, dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL((decode_matrix_kernel<4, FUSED, 4, PAGED, CAUSAL>), grid, dim3(256), 0, stream, p);
  }
}

}  // namespace

hipError_t launch_decode_matrix(const DecodeParams& p, hipStream_t stream) {
  const bool paged = p.pg.table != nullptr;
  if (p.n_tok > 1) paged ? launch_nb<false, true, true>(p, stream) : launch_nb<false, false, true>(p, stream);
  else if (p.fused) paged ? launch_nb<true, true, false>(p, stream) : launch_nb<true, false, false>(p, stream);
  else paged ? launch_nb<false, true, false>(p, stream) : launch_nb<false, false, false>(p, stream);
  return hipGetLastError();
}

namespace {
template <bool FUSED, bool PAGED, bool CAUSAL>
hipError_t occupancy(int k, int* n) {
  if (k == 0)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        n, decode_matrix_kernel<1, FUSED, kMatrixWaves1, PAGED, CAUSAL>, kMatrixWaves1 * 64, 0);
  if (k == 1)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, decode_matrix_kernel<2, FUSED, 4, PAGED, CAUSAL>, 256, 0);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, decode_matrix_kernel<4, FUSED, 4, PAGED, CAUSAL>, 256, 0);
}
}  // namespace

int matrix_waves(int G) { return G <= 16 ? kMatrixWaves1 : 4; }

// kind: 0 one-token, 1 fused step, 2 paged, 3 paged fused step, 4 multi-token,
// 5 paged multi-token (the multi-token append is its own launch: never fused).
// The answer depends only on the kernel and the architecture, so it is kept
// once per process (relaxed atomics: concurrent first calls store the same value).
int matrix_workgroups_per_cu(int G, bool fused, bool paged, bool causal) {
  static std::atomic<int> cached[6][3] = {};
  const int k = G <= 16 ? 0 : (G <= 32 ? 1 : 2);
  const int kind = causal ? (paged ? 5 : 4) : (paged ? 2 : 0) + (fused ? 1 : 0);
  std::atomic<int>& c = cached[kind][k];
  const int known = c.load(std::memory_order_relaxed);
  if (known > 0) return known;
  int n = 0;
  hipError_t e;
  switch (kind) {
    case 0: e = occupancy<false, false, false>(k, &n); break;
    case 1: e = occupancy<true, false, false>(k, &n); break;
    case 2: e = occupancy<false, true, false>(k, &n); break;
    case 3: e = occupancy<true, true, false>(k, &n); break;
    case 4: e = occupancy<false, false, true>(k, &n); break;
    default: e = occupancy<false, true, true>(k, &n); break;
  }
  if (e != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 0;
  }
  c.store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace gqa
