// Streaming read of a device buffer: the read bandwidth this part sustains,
// against which the decode kernels' HBM roofline can be stated besides the
// nominal 8 TB/s (the pages call decode memory-bound: "LLM inference 05", the
// decode phase; MQA review §2.4, the K/V re-read of the incremental step).
//
// The grid is persistent, one 512-thread workgroup per compute unit as for
// the stream kernel. Workgroup w reads the contiguous range [w n / P,
// (w + 1) n / P) of the buffer's n 16-byte chunks with non-temporal buffer
// loads (the decode kernels' form), eight per thread in flight; its buffer
// resource covers exactly that range, so the tail needs no test. It leaves
// the sum of every 32-bit word it read (mod 2^32) in sink[w]: the loads
// cannot be dropped, and the sink's total tells whether every word was read
// once.
#include "gqa_internal.hpp"

namespace gqa {
namespace {

constexpr int kReadThreads = 512;
constexpr int kReadUnroll = 8;
constexpr int kReadCpol = 2;  // NT: each byte is read once

__global__ __launch_bounds__(kReadThreads, 1) void read_bandwidth_kernel(const unsigned char* src, long long n16,
                                                                          uint32_t* sink) {
  __shared__ uint32_t s_part[kReadThreads / 64];
  const long long P = gridDim.x;
  const long long begin = n16 * blockIdx.x / P;
  const long long end = n16 * (blockIdx.x + 1) / P;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(src) + begin * 16, 0, int((end - begin) * 16), kBufferWord3);
  uint32_t acc = 0;
  for (int base = 0; base < int(end - begin); base += kReadThreads * kReadUnroll) {
    u32x4v v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      v[u] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(
                                            r, (base + u * kReadThreads + int(threadIdx.x)) * 16, 0, kReadCpol));
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc += v[u][0] + v[u][1] + v[u][2] + v[u][3];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < kReadThreads / 64; ++i) t += s_part[i];
    sink[blockIdx.x] = t;
  }
}

}  // namespace

hipError_t launch_read_bandwidth(const void* src, size_t bytes, uint32_t* sink, int workgroups,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(read_bandwidth_kernel, dim3(workgroups), dim3(kReadThreads), 0, stream,
                     static_cast<const unsigned char*>(src), (long long)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace gqa
