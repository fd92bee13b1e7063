// Linear projections around the decode step: the query, key and value
// projections of the new token before the append, and the output projection
// after the attention ("Fast Transformer Decoding: One Write-Head is All You
// Need" review, §2.4 incremental multi-head attention: q, k and v are the
// token's vector times P_q, P_k, P_v, and y is the attention output times
// P_o; §3 drops the head axis of P_k and P_v for MQA).
//
// Each projection is y[r][o] = sum_k w[o][k] * x[r][k] for the decode batch
// (r < rows <= 64): a matrix-vector product per sequence, bound by reading w
// once from HBM. The same 16x16x32 bf16 MFMA as the score step applies with
// the weights as the A operand and the batch as B:
//
//   C[o][r] = sum_k w[o][k] * x[r][k]     A = 16 weight rows x 32 k, B = x^T
//
// Lane (n = l%16, q = l/16) needs 16 bytes of weight row o0 + n at k = 32s +
// 8q for each k-step s. Read from the [n_out][n_in] matrix those are sixteen
// 64-byte pieces of rows n_in*2 bytes apart, which streams at about half the
// HBM rate; so the weights are packed once (pack_weight_kernel) in exactly
// that order: tile (block, s) is 1 KiB, lane l's 16 bytes at offset 16*l,
// tiles of one block consecutive in s, and one wave load reads one
// contiguous KiB. Rows past n_out and k past n_in are zero in the packing.
// A workgroup owns one or two blocks of 16 output features; its four waves
// take every fourth k-step and their partial blocks are summed through LDS.
// Batch row 16*nb + n is read for the same k range and serves both blocks.
// Several weight matrices (the query, key and value projections of one
// token) go through one launch as consecutive ranges of workgroups, so that
// the narrow key and value projections share the grid with the wide query
// projection; a matrix with an odd block count ends in a workgroup with one.
#include "gqa_internal.hpp"

namespace gqa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLinWaves = 4;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// MB blocks of 16 output features per workgroup share each batch load (MB = 2
// measured faster from 16 batch rows up, MB = 1 below).
template <int NB, int MB>
__global__ __launch_bounds__(kLinWaves * 64) void linear_bf16_kernel(LinearParams p) {
  constexpr int UNROLL = NB * MB <= 2 ? 8 : 4;  // k-steps whose loads are in flight together
  __shared__ float red[kLinWaves][NB][16 * MB][17];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n16 = lane & 15;
  const int q4 = lane >> 4;

  // which matrix and which MB blocks of 16 output features
  int seg = 0, grp = blockIdx.x;
  while (seg + 1 < p.nseg && grp >= (p.blocks[seg] + MB - 1) / MB) {
    grp -= (p.blocks[seg] + MB - 1) / MB;
    ++seg;
  }
  const int n_out = p.n_out[seg];
  const int blk = grp * MB;
  const int nblk = min(MB, p.blocks[seg] - blk);
  const int o0 = blk * 16;
  const int nsteps = (p.n_in + 31) / 32;
  const u32x4* wtile = reinterpret_cast<const u32x4*>(p.w[seg]) + size_t(blk) * nsteps * 64 + lane;

  f32x4 acc[MB][NB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[m][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int s0 = w; s0 < nsteps; s0 += kLinWaves * UNROLL) {
    u32x4 wa[UNROLL][MB];
    u32x4 xb[UNROLL][NB];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int s = s0 + u * kLinWaves;
      const int k = 32 * s + 8 * q4;
      const bool k_ok = s < nsteps && k < p.n_in;  // n_in is a multiple of 8
#pragma unroll
      for (int m = 0; m < MB; ++m)
        wa[u][m] = (s < nsteps && m < nblk) ? __builtin_nontemporal_load(wtile + (size_t(m) * nsteps + s) * 64)
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
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wa[u][m]), as_bf16x8(xb[u][nb]), acc[m][nb],
                                                               0, 0, 0);
  }

  // lane (n, q) holds C[4q + i][n] of block m: output feature o0 + 16m + 4q + i, batch row 16*nb + n
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w][nb][16 * m + 4 * q4 + i][n16] = acc[m][nb][i];
  __syncthreads();
  uint16_t* y = p.y[seg];
  constexpr int PER_NB = 16 * 16 * MB;  // outputs of one batch block
  for (int idx = threadIdx.x; idx < NB * PER_NB; idx += kLinWaves * 64) {
    const int nb = idx / PER_NB, rem = idx - nb * PER_NB;
    const int rr = rem / (16 * MB), o = rem - rr * (16 * MB);  // consecutive threads: consecutive outputs
    const int r = 16 * nb + rr;
    float v = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kLinWaves; ++ww) v += red[ww][nb][o][rr];
    if (r < p.rows && o0 + o < n_out) y[size_t(r) * n_out + o0 + o] = f32_to_bf16(v);
  }
}

// Pack w [n_out][n_in] (bf16) into the MFMA tile order above: one thread per
// 16-byte lane slot of the packed array, zero where the row or k is out of
// range.
__global__ __launch_bounds__(256) void pack_weight_kernel(uint16_t* dst, const uint16_t* src, int n_out, int n_in,
                                                          size_t slots) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= slots) return;
  const int nsteps = (n_in + 31) / 32;
  const int lane = int(i & 63);
  const size_t tile = i >> 6;
  const int s = int(tile % nsteps);
  const size_t blk = tile / nsteps;
  const size_t o = blk * 16 + (lane & 15);
  const int k = 32 * s + 8 * (lane >> 4);
  u32x4 v = {0u, 0u, 0u, 0u};
  if (o < size_t(n_out) && k < n_in) {
    const uint16_t* row = src + o * size_t(n_in) + k;
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = (k + j < n_in) ? row[j] : uint16_t(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = uint32_t(e[2 * j]) | (uint32_t(e[2 * j + 1]) << 16);
  }
  reinterpret_cast<u32x4*>(dst)[i] = v;
}

}  // namespace

size_t packed_weight_bytes(int n_out, int n_in) {
  return size_t((n_out + 15) / 16) * 16 * size_t((n_in + 31) / 32) * 32 * sizeof(uint16_t);
}

hipError_t launch_pack_weight(void* dst, const void* src, int n_out, int n_in, hipStream_t stream) {
  const size_t slots = packed_weight_bytes(n_out, n_in) / 16;
  const size_t blocks = (slots + 255) / 256;
  hipLaunchKernelGGL(pack_weight_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, static_cast<uint16_t*>(dst),
                     static_cast<const uint16_t*>(src), n_out, n_in, slots);
  return hipGetLastError();
}

hipError_t launch_linear(const LinearParams& p, hipStream_t stream) {
  const int mb = p.rows >= 16 ? 2 : 1;
  int groups = 0;
  for (int s = 0; s < p.nseg; ++s) groups += (p.blocks[s] + mb - 1) / mb;
  const dim3 grid(groups), block(kLinWaves * 64);
  if (mb == 1) hipLaunchKernelGGL((linear_bf16_kernel<1, 1>), grid, block, 0, stream, p);
  else if (p.rows <= 16) hipLaunchKernelGGL((linear_bf16_kernel<1, 2>), grid, block, 0, stream, p);
  else if (p.rows <= 32) hipLaunchKernelGGL((linear_bf16_kernel<2, 2>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((linear_bf16_kernel<4, 2>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
