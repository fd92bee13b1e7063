// Internal declarations shared by the gfx950 kernels and the C-ABI shim.
//
// Workspace layout (one buffer, caller-owned, see gqa_decode_workspace_size):
//   [counters]  int32  [b*h]                      zero between calls
//   [ml]        float  [b*h][nch_stride][2]       (running max m, sum l) per chunk
//   [o]         float  [b*h][nch_stride][d_v]     unnormalised partial output
// Each region starts on a 256-byte boundary. nch_stride = ceil(max_len / 64),
// the largest chunk count any chunk size (a multiple of 64) can produce.
// The softmax state is kept in base-2 units: m is the max of scale*log2(e)*q.k.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

constexpr int kMinChunk = 64;     // chunk granularity (positions)
constexpr int kMaxChunk = 65536;  // largest chunk the shim accepts
constexpr int kThreads = 256;     // workgroup size of both decode kernels
constexpr int kWaves = kThreads / 64;

struct AppendParams {
  void* k_cache;
  void* v_cache;
  const void* k_new;
  const void* v_new;
  int32_t* lens;
  int g, d_k, d_v, cap;
};

struct DecodeParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* lens;
  int* ws_cnt;
  float* ws_ml;
  float* ws_o;
  int b, h, g, G, d, cap, max_len;
  int chunk;       // positions per workgroup
  int nch_stride;  // chunk slots per (sequence, head) in the workspace
  float scale_log2;  // scale * log2(e)
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline int nch_stride_for(int max_len) {
  const int n = (max_len + kMinChunk - 1) / kMinChunk;
  return n > 0 ? n : 1;
}

struct WorkspaceLayout {
  size_t cnt_off, ml_off, o_off, total;
};

inline WorkspaceLayout workspace_layout(int b, int h, int d_v, int max_len) {
  const size_t rows = size_t(b) * size_t(h);
  const size_t nch = size_t(nch_stride_for(max_len));
  WorkspaceLayout w;
  w.cnt_off = 0;
  w.ml_off = align256(rows * sizeof(int));
  w.o_off = w.ml_off + align256(rows * nch * 2 * sizeof(float));
  w.total = w.o_off + align256(rows * nch * size_t(d_v) * sizeof(float));
  return w;
}

// Launchers (defined next to their kernels). Return the hipError_t of the
// launch.
hipError_t launch_append(const AppendParams& p, int b, int dtype, hipStream_t stream);
hipError_t launch_decode_vector(const DecodeParams& p, int dtype, int heads_per_block,
                                hipStream_t stream);
hipError_t launch_decode_matrix(const DecodeParams& p, hipStream_t stream);

// Vector-path head block for G query heads per KV head: the smallest power of
// two >= G, capped at 8 (larger groups use several head blocks).
inline int vector_heads_per_block(int G) {
  if (G <= 1) return 1;
  if (G <= 2) return 2;
  if (G <= 4) return 4;
  return 8;
}

}  // namespace gqa

#if defined(__HIPCC__)
namespace gqa {

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
// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15-i within 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float xor_shuffle(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}

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

// Combine two split-softmax states (m in base-2 units); the result is written
// to (m, l). Either state may be empty (m = -inf, l = 0, acc = 0).
struct MergeWeights {
  float a, b;
};
__device__ __forceinline__ MergeWeights merge_weights(float m1, float m2, float& m_out) {
  const float M = fmaxf(m1, m2);
  const float sub = (M == kNegInf) ? 0.0f : M;
  m_out = M;
  return {fast_exp2(m1 - sub), fast_exp2(m2 - sub)};
}

// ------------------------------------------------------- split finishing
// Called by every thread of a workgroup once its combined state for query
// heads [i0, i0 + nh) of sequence s over chunk c is in LDS:
//   sm_m[nh], sm_l[nh]: base-2 running max and sum; sm_o[nh][d]: unnormalised
//   output. n_valid is the number of chunks of this sequence that hold
//   positions.
// With one chunk the output is written directly. Otherwise the state goes to
// the workspace, and the last workgroup of the (s, i0) group to finish
// (an atomic ticket, released and acquired with device-scope fences) merges
// every chunk's state and writes the output, then re-zeroes the ticket.
template <typename TOut>
__device__ void finish_chunk(const DecodeParams& p, int s, int i0, int nh, int c, int n_valid,
                             const float* sm_m, const float* sm_l, const float* sm_o,
                             int* sm_flag) {
  const int tid = threadIdx.x;
  const int d = p.d;
  TOut* out = static_cast<TOut*>(p.out);
  const size_t out_row0 = (size_t(s) * p.h + i0) * d;
  if (n_valid == 1) {
    for (int idx = tid; idx < nh * d; idx += kThreads) {
      const float l = sm_l[idx / d];
      const float v = l > 0.0f ? sm_o[idx] / l : 0.0f;
      if constexpr (sizeof(TOut) == 2) out[out_row0 + idx] = f32_to_bf16(v);
      else out[out_row0 + idx] = v;
    }
    return;
  }
  const size_t row0 = size_t(s) * p.h + i0;
  const size_t stride = size_t(p.nch_stride);
  for (int idx = tid; idx < nh * d; idx += kThreads) {
    const int hh = idx / d, dd = idx - hh * d;
    p.ws_o[((row0 + hh) * stride + c) * d + dd] = sm_o[idx];
  }
  for (int hh = tid; hh < nh; hh += kThreads) {
    p.ws_ml[((row0 + hh) * stride + c) * 2 + 0] = sm_m[hh];
    p.ws_ml[((row0 + hh) * stride + c) * 2 + 1] = sm_l[hh];
  }
  __threadfence();  // release this workgroup's partials device-wide
  __syncthreads();
  if (tid == 0) {
    const int prev = atomicAdd(&p.ws_cnt[row0], 1);
    *sm_flag = (prev == n_valid - 1);
  }
  __syncthreads();
  if (!*sm_flag) return;
  __threadfence();  // acquire the other workgroups' partials
  for (int idx = tid; idx < nh * d; idx += kThreads) {
    const int hh = idx / d, dd = idx - hh * d;
    const size_t base = (row0 + hh) * stride;
    float M = kNegInf;
    for (int cc = 0; cc < n_valid; ++cc) M = fmaxf(M, p.ws_ml[(base + cc) * 2]);
    const float sub = (M == kNegInf) ? 0.0f : M;
    float num = 0.0f, den = 0.0f;
    for (int cc = 0; cc < n_valid; ++cc) {
      const float wgt = fast_exp2(p.ws_ml[(base + cc) * 2] - sub);
      num += wgt * p.ws_o[(base + cc) * d + dd];
      den += wgt * p.ws_ml[(base + cc) * 2 + 1];
    }
    const float v = den > 0.0f ? num / den : 0.0f;
    if constexpr (sizeof(TOut) == 2) out[out_row0 + idx] = f32_to_bf16(v);
    else out[out_row0 + idx] = v;
  }
  if (tid == 0) p.ws_cnt[row0] = 0;
}

// Zero output rows of a sequence that attends no positions.
template <typename TOut>
__device__ void write_zero_rows(const DecodeParams& p, int s, int i0, int nh) {
  TOut* out = static_cast<TOut*>(p.out);
  const size_t row0 = (size_t(s) * p.h + i0) * p.d;
  for (int idx = threadIdx.x; idx < nh * p.d; idx += kThreads) out[row0 + idx] = TOut(0);
}

// Effective attended length: lens clamped to [0, max_len].
__device__ __forceinline__ int attended_len(const DecodeParams& p, int s) {
  int L = p.lens[s];
  L = L < 0 ? 0 : L;
  return L > p.max_len ? p.max_len : L;
}

}  // namespace gqa
#endif  // __HIPCC__
