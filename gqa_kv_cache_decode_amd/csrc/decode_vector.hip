// Vector-ALU split-K decode attention (every supported dtype and head dim).
//
// Computes, per sequence s and query head i with KV head j = floor(i / G),
//   out[s][i] = sum_t softmax_t(scale * q[s][i] . K[s][j][t]) V[s][j][t]
// (MQA review §2.1 Dot-Product Attention applied per head, with the cache of
// §2.4 / §3 and the contiguous head groups of the TF2 GQA lesson).
//
// Work decomposition: one workgroup per (position chunk, KV head, head block,
// sequence). A head block is up to 8 query heads of one group, so each K/V
// row fetched from HBM is used by all of them. A K/V row is split over
// R = row_bytes / 16 consecutive lanes, each holding one 16-byte column, and
// each wave load instruction covers 64 / R consecutive rows (1 KiB,
// contiguous). Dot products are summed across the R lanes with DPP row
// operations; every lane group keeps its own online-softmax state (running
// max, sum, unnormalised output) in base 2, and the groups, then the four
// waves (through LDS), are merged at the end. finish_chunk then writes the
// output or the chunk's partial state and merges the chunks.
#include "gqa_internal.hpp"

namespace gqa {
namespace {

template <typename T>
__device__ __forceinline__ void widen16(const uint4& r, float* f) {
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

template <typename T, int D, int HB>
__global__ __launch_bounds__(kThreads) void decode_vector_kernel(DecodeParams p) {
  constexpr int VEC = 16 / int(sizeof(T));  // elements per 16-byte column
  constexpr int R = D / VEC;                // lanes per row
  static_assert(R >= 1 && R <= 64 && (R & (R - 1)) == 0, "row must be 16..1024 bytes");
  constexpr int RPW = 64 / R;               // rows per wave load
  constexpr int U = (HB >= 8 && VEC == 8) ? 2 : 4;  // loads in flight per lane
  constexpr int ROWS_IT = kWaves * RPW * U;

  __shared__ float sm_m[kWaves][HB];
  __shared__ float sm_l[kWaves][HB];
  __shared__ float sm_o[kWaves][HB][D];
  __shared__ float fin_m[HB];
  __shared__ float fin_l[HB];
  __shared__ float fin_o[HB][D];
  __shared__ int s_flag;

  const int c = blockIdx.x;
  const int nhb = (p.G + HB - 1) / HB;
  const int j = blockIdx.y / nhb;
  const int hb = blockIdx.y - j * nhb;
  const int s = blockIdx.z;
  const int i0 = j * p.G + hb * HB;
  const int nh = min(HB, p.G - hb * HB);
  const int L = attended_len(p, s);
  if (L == 0) {
    if (c == 0) write_zero_rows<T>(p, s, i0, nh);
    return;
  }
  const int n_valid = (L + p.chunk - 1) / p.chunk;
  if (c >= n_valid) return;
  const int t_begin = c * p.chunk;
  const int t_end = min(L, t_begin + p.chunk);

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int col = lane % R;
  const int rg = lane / R;

  // Query rows of the head block, widened and pre-multiplied by scale*log2(e).
  float qf[HB][VEC];
  const T* qrow = static_cast<const T*>(p.q) + (size_t(s) * p.h + i0) * D + col * VEC;
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    if (hh < nh) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qrow + size_t(hh) * D);
      widen16<T>(raw, qf[hh]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) qf[hh][e] *= p.scale_log2;
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) qf[hh][e] = 0.0f;
    }
  }

  float m[HB], l[HB], acc[HB][VEC];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    m[hh] = kNegInf;
    l[hh] = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[hh][e] = 0.0f;
  }

  const size_t kv_head = size_t(s) * p.g + j;
  const T* kbase = static_cast<const T*>(p.k_cache) + kv_head * p.cap * D + col * VEC;
  const T* vbase = static_cast<const T*>(p.v_cache) + kv_head * p.cap * D + col * VEC;

  for (int base = t_begin + w * RPW * U; base < t_end; base += ROWS_IT) {
    uint4 kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + u * RPW + rg;
      ok[u] = t < t_end;
      if (ok[u]) {
        kr[u] = *reinterpret_cast<const uint4*>(kbase + size_t(t) * D);
        vr[u] = *reinterpret_cast<const uint4*>(vbase + size_t(t) * D);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
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
        sc[u][hh] = ok[u] ? part : kNegInf;
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
      const float mn = fmaxf(m[hh], mx);
      const float sub = (mn == kNegInf) ? 0.0f : mn;
      const float alpha = fast_exp2(m[hh] - sub);
      m[hh] = mn;
      float pu[U];
      float psum = 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        pu[u] = fast_exp2(sc[u][hh] - sub);
        psum += pu[u];
      }
      l[hh] = fmaf(l[hh], alpha, psum);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float a = acc[hh][e] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) a = fmaf(pu[u], vf[u][e], a);
        acc[hh][e] = a;
      }
    }
  }

  // Merge the lane groups of the wave (same column, different rows).
#pragma unroll
  for (int off = R; off < 64; off <<= 1) {
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      const float mo = xor_shuffle(m[hh], off);
      const float lo = xor_shuffle(l[hh], off);
      float mn;
      const MergeWeights wt = merge_weights(m[hh], mo, mn);
      l[hh] = l[hh] * wt.a + lo * wt.b;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float ao = xor_shuffle(acc[hh][e], off);
        acc[hh][e] = acc[hh][e] * wt.a + ao * wt.b;
      }
      m[hh] = mn;
    }
  }
  if (rg == 0) {
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm_o[w][hh][col * VEC + e] = acc[hh][e];
      if (col == 0) {
        sm_m[w][hh] = m[hh];
        sm_l[w][hh] = l[hh];
      }
    }
  }
  __syncthreads();
  // Merge the four waves.
  for (int idx = threadIdx.x; idx < HB * D; idx += kThreads) {
    const int hh = idx / D, dd = idx - hh * D;
    float M = sm_m[0][hh];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, sm_m[ww][hh]);
    const float sub = (M == kNegInf) ? 0.0f : M;
    float o = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
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
  finish_chunk<T>(p, s, i0, nh, c, n_valid, fin_m, fin_l, &fin_o[0][0], &s_flag);
}

template <typename T, int D>
hipError_t launch_d(const DecodeParams& p, int hb, hipStream_t stream) {
  const int n_chunks = (p.max_len + p.chunk - 1) / p.chunk;
  const int nhb = (p.G + hb - 1) / hb;
  const dim3 grid(n_chunks > 0 ? n_chunks : 1, p.g * nhb, p.b);
  switch (hb) {
    case 1: hipLaunchKernelGGL((decode_vector_kernel<T, D, 1>), grid, dim3(kThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_vector_kernel<T, D, 2>), grid, dim3(kThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_vector_kernel<T, D, 4>), grid, dim3(kThreads), 0, stream, p); break;
    default: hipLaunchKernelGGL((decode_vector_kernel<T, D, 8>), grid, dim3(kThreads), 0, stream, p); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const DecodeParams& p, int hb, hipStream_t stream) {
  switch (p.d) {
    case 16: return launch_d<T, 16>(p, hb, stream);
    case 32: return launch_d<T, 32>(p, hb, stream);
    case 64: return launch_d<T, 64>(p, hb, stream);
    case 128: return launch_d<T, 128>(p, hb, stream);
    case 256: return launch_d<T, 256>(p, hb, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_vector(const DecodeParams& p, int dtype, int heads_per_block,
                                hipStream_t stream) {
  if (dtype == 0) return launch_t<float>(p, heads_per_block, stream);
  return launch_t<uint16_t>(p, heads_per_block, stream);
}

}  // namespace gqa
