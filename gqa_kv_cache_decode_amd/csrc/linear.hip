// Linear projections around the decode step: the query, key and value
// projections of the new token before the append, and the output projection
// after the attention ("Fast Transformer Decoding: One Write-Head is All You
// Need" review, §2.4 incremental multi-head attention: q, k and v are the
// token's vector times P_q, P_k, P_v, and y is the attention output times
// P_o; §3 drops the head axis of P_k and P_v for MQA).
//
// Each projection is y[r][o] = sum_k x[r][k] * w[o][k] for the decode batch
// (r < rows <= 64): a matrix-vector product per sequence, bound by reading w
// once from HBM. w is stored output-major, [n_out][n_in] (row o holds the
// weights of output feature o), so the same 16x16x32 bf16 MFMA as the score
// step applies with the weights as the A operand and the batch as B:
//
//   C[o][r] = sum_k w[o][k] * x[r][k]     A = 16 weight rows x 32 k, B = x^T
//
// Lane (n = l%16, q = l/16) loads 16 bytes of weight row o0 + n at k = 32s +
// 8q for each k-step s, and the same k range of batch row 16*nb + n. A
// workgroup owns 16 output features; its four waves take every fourth k-step
// and their 16 x 16 partial blocks are summed through LDS. Several weight
// matrices (the query, key and value projections of one token) go through
// one launch as consecutive ranges of output blocks, so that the narrow key
// and value projections share the grid with the wide query projection.
#include "gqa_internal.hpp"

namespace gqa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLinWaves = 4;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int NB>
__global__ __launch_bounds__(kLinWaves * 64) void linear_bf16_kernel(LinearParams p) {
  constexpr int UNROLL = NB <= 2 ? 8 : 4;  // k-steps whose loads are in flight together
  __shared__ float red[kLinWaves][NB][16][17];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n16 = lane & 15;
  const int q4 = lane >> 4;

  // which matrix and which 16 output features
  int seg = 0, blk = blockIdx.x;
  while (seg + 1 < p.nseg && blk >= p.blocks[seg]) {
    blk -= p.blocks[seg];
    ++seg;
  }
  const int n_out = p.n_out[seg];
  const int o0 = blk * 16;
  const int orow = o0 + n16;
  const uint16_t* wrow = p.w[seg] + size_t(orow < n_out ? orow : n_out - 1) * p.n_in;
  const bool orow_ok = orow < n_out;

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int nsteps = (p.n_in + 31) / 32;
  for (int s0 = w; s0 < nsteps; s0 += kLinWaves * UNROLL) {
    u32x4 wa[UNROLL];
    u32x4 xb[UNROLL][NB];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int s = s0 + u * kLinWaves;
      const int k = 32 * s + 8 * q4;
      const bool k_ok = s < nsteps && k < p.n_in;  // n_in is a multiple of 8
      wa[u] = (k_ok && orow_ok) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow + k))
                                : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int r = 16 * nb + n16;
        xb[u][nb] = (k_ok && r < p.rows) ? *reinterpret_cast<const u32x4*>(p.x + size_t(r) * p.n_in + k)
                                         : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wa[u]), as_bf16x8(xb[u][nb]), acc[nb], 0, 0, 0);
  }

  // lane (n, q) holds C[4q + i][n]: output feature o0 + 4q + i, batch row 16*nb + n
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[w][nb][4 * q4 + i][n16] = acc[nb][i];
  __syncthreads();
  uint16_t* y = p.y[seg];
  for (int idx = threadIdx.x; idx < NB * 256; idx += kLinWaves * 64) {
    const int nb = idx >> 8, rem = idx & 255;
    const int r = 16 * nb + (rem >> 4), o = rem & 15;  // consecutive threads: consecutive outputs
    float v = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kLinWaves; ++ww) v += red[ww][nb][o][rem >> 4];
    if (r < p.rows && o0 + o < n_out) y[size_t(r) * n_out + o0 + o] = f32_to_bf16(v);
  }
}

}  // namespace

hipError_t launch_linear(const LinearParams& p, hipStream_t stream) {
  int blocks = 0;
  for (int s = 0; s < p.nseg; ++s) blocks += p.blocks[s];
  const dim3 grid(blocks), block(kLinWaves * 64);
  if (p.rows <= 16) hipLaunchKernelGGL(linear_bf16_kernel<1>, grid, block, 0, stream, p);
  else if (p.rows <= 32) hipLaunchKernelGGL(linear_bf16_kernel<2>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(linear_bf16_kernel<4>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
