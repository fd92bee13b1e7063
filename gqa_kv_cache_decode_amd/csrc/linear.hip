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
// A workgroup owns one to three consecutive blocks of 16 output features
// (the launch's blocks split evenly over one workgroup per compute unit); its
// eight waves take every eighth k-step and their partial blocks are summed
// through LDS. Batch row 16*nb + n is read for the same k range and serves
// all the workgroup's blocks. Several weight matrices (the query, key and
// value projections of one token) go through one launch as consecutive
// blocks, so that the narrow key and value projections share the grid with
// the wide query projection; a workgroup may hold blocks of two of them.
#include "gqa_internal.hpp"

namespace gqa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLinWaves = 8;  // waves per workgroup (8 measured 2-10 % faster than 4)

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Workgroup w owns the consecutive output blocks [b0, b1) = [w*B/P,
// (w+1)*B/P) of the launch's B blocks of 16 features (all segments in a row;
// a block of any segment multiplies the same x), at most MB of them, so every
// workgroup reads the same weight bytes within one block and each batch load
// serves all its blocks.
template <int NB, int MB, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void linear_bf16_kernel(LinearParams p) {
  constexpr int UNROLL = NB * MB <= 2 ? 8 : 4;  // k-steps whose loads are in flight together
  __shared__ float red[WAVES][NB][16 * MB][17];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n16 = lane & 15;
  const int q4 = lane >> 4;

  int total = 0;
  for (int sg = 0; sg < p.nseg; ++sg) total += p.blocks[sg];
  const int b0 = int((long long)blockIdx.x * total / gridDim.x);
  const int nblk = int((long long)(blockIdx.x + 1) * total / gridDim.x) - b0;  // 1 .. MB
  const int nsteps = (p.n_in + 31) / 32;

  // the weight tiles of each block (blocks past nblk repeat the last one and are not read)
  const u32x4* wt[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    int blk = min(b0 + m, total - 1), sg = 0;
    while (sg + 1 < p.nseg && blk >= p.blocks[sg]) {
      blk -= p.blocks[sg];
      ++sg;
    }
    wt[m] = reinterpret_cast<const u32x4*>(p.w[sg]) + size_t(blk) * nsteps * 64 + lane;
  }

  f32x4 acc[MB][NB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[m][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int s0 = w; s0 < nsteps; s0 += WAVES * UNROLL) {
    u32x4 wa[UNROLL][MB];
    u32x4 xb[UNROLL][NB];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int s = s0 + u * WAVES;
      const int k = 32 * s + 8 * q4;
      const bool k_ok = s < nsteps && k < p.n_in;  // n_in is a multiple of 8
#pragma unroll
      for (int m = 0; m < MB; ++m)
        wa[u][m] = (s < nsteps && m < nblk) ? __builtin_nontemporal_load(wt[m] + size_t(s) * 64)
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

  // lane (n, q) holds C[4q + i][n] of block m: its feature 4q + i, batch row 16*nb + n
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w][nb][16 * m + 4 * q4 + i][n16] = acc[m][nb][i];
  __syncthreads();
  constexpr int PER_NB = 16 * 16 * MB;  // outputs of one batch block
  for (int idx = threadIdx.x; idx < NB * PER_NB; idx += WAVES * 64) {
    const int nb = idx / PER_NB, rem = idx - nb * PER_NB;
    const int rr = rem / (16 * MB), o = rem - rr * (16 * MB);  // consecutive threads: consecutive outputs
    const int m = o >> 4, r = 16 * nb + rr;
    float v = 0.0f;
#pragma unroll
    for (int ww = 0; ww < WAVES; ++ww) v += red[ww][nb][o][rr];
    if (m < nblk && r < p.rows) {
      int blk = b0 + m, sg = 0;
      while (sg + 1 < p.nseg && blk >= p.blocks[sg]) {
        blk -= p.blocks[sg];
        ++sg;
      }
      const int f = blk * 16 + (o & 15), no = p.n_out[sg];
      if (f < no) p.y[sg][size_t(r) * no + f] = f32_to_bf16(v);
    }
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

template <int NB, int W>
void launch_mb(const LinearParams& p, int mb, dim3 g, hipStream_t stream) {
  const dim3 block(W * 64);
  if (mb == 1) hipLaunchKernelGGL((linear_bf16_kernel<NB, 1, W>), g, block, 0, stream, p);
  else if (mb == 2) hipLaunchKernelGGL((linear_bf16_kernel<NB, 2, W>), g, block, 0, stream, p);
  else hipLaunchKernelGGL((linear_bf16_kernel<NB, 3, W>), g, block, 0, stream, p);
}

template <int W>
void launch_w(const LinearParams& p, int mb, dim3 g, hipStream_t stream) {
  if (p.rows <= 16) launch_mb<1, W>(p, mb, g, stream);
  else if (p.rows <= 32) launch_mb<2, W>(p, mb, g, stream);
  else launch_mb<4, W>(p, mb, g, stream);
}

hipError_t launch_linear(const LinearParams& p, hipStream_t stream) {
  int total = 0;
  for (int s = 0; s < p.nseg; ++s) total += p.blocks[s];
  // one workgroup per compute unit with up to three blocks each; past that,
  // as many workgroups of three blocks as needed
  const int cus = 256;
  int grid = total <= cus ? total : (total <= 3 * cus ? cus : (total + 2) / 3);
  const int mb = (total + grid - 1) / grid;
  launch_w<kLinWaves>(p, mb, dim3(grid), stream);
  return hipGetLastError();
}

}  // namespace gqa
