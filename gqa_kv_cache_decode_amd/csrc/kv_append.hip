// Append one token's K and V rows per sequence to the cache, then grow the
// length by one ("LLM inference 05" notes: push K, push V before attending;
// MQA review §2.4 / §3: the new row is concatenated on the position axis).
//
// One workgroup per sequence: it reads lens[s] once, copies the g new K rows
// and g new V rows into slot lens[s] with 16-byte (or narrower) moves, and
// only after a barrier writes lens[s] + 1, so every thread used the old
// length. A length outside [0, cap) leaves the sequence untouched.
#include "gqa_internal.hpp"

namespace gqa {
namespace {

// Copy n_bytes from src to dst with the widest unit that divides both the
// size and the alignment (caches are contiguous rows, so rows of 16-byte
// multiples move as uint4).
__device__ __forceinline__ void copy_row_bytes(char* dst, const char* src, int n_bytes) {
  if ((n_bytes & 15) == 0 && ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15) == 0) {
    for (int i = threadIdx.x; i < (n_bytes >> 4); i += blockDim.x)
      reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
  } else if ((n_bytes & 3) == 0 && ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 3) == 0) {
    for (int i = threadIdx.x; i < (n_bytes >> 2); i += blockDim.x)
      reinterpret_cast<uint32_t*>(dst)[i] = reinterpret_cast<const uint32_t*>(src)[i];
  } else {
    for (int i = threadIdx.x; i < (n_bytes >> 1); i += blockDim.x)
      reinterpret_cast<uint16_t*>(dst)[i] = reinterpret_cast<const uint16_t*>(src)[i];
  }
}

__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p, int esize) {
  const int s = blockIdx.x;
  __shared__ int s_pos;
  if (threadIdx.x == 0) s_pos = p.lens[s];
  __syncthreads();
  const int pos = s_pos;
  if (pos < 0 || pos >= p.cap) return;  // precondition violated: change nothing
  const int kb = p.d_k * esize, vb = p.d_v * esize;
  for (int j = 0; j < p.g; ++j) {
    const size_t head = size_t(s) * p.g + j;
    char* kdst = static_cast<char*>(p.k_cache) + (head * p.cap + pos) * kb;
    char* vdst = static_cast<char*>(p.v_cache) + (head * p.cap + pos) * vb;
    copy_row_bytes(kdst, static_cast<const char*>(p.k_new) + head * kb, kb);
    copy_row_bytes(vdst, static_cast<const char*>(p.v_new) + head * vb, vb);
  }
  __syncthreads();
  if (threadIdx.x == 0) p.lens[s] = pos + 1;
}

}  // namespace

hipError_t launch_append(const AppendParams& p, int b, int dtype, hipStream_t stream) {
  const int esize = dtype == 0 ? 4 : 2;
  // one wave per 16-byte unit of the widest row, at least one wave, at most 256 threads
  int units = ((p.d_k > p.d_v ? p.d_k : p.d_v) * esize + 15) / 16;
  int threads = ((units + 63) / 64) * 64;
  if (threads < 64) threads = 64;
  if (threads > 256) threads = 256;
  hipLaunchKernelGGL(kv_append_kernel, dim3(b), dim3(threads), 0, stream, p, esize);
  return hipGetLastError();
}

}  // namespace gqa
