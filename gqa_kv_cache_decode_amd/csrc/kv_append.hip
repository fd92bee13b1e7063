// Append one token's K and V rows per sequence to the cache, then grow the
// length by one ("LLM inference 05" notes: push K, push V before attending;
// MQA review §2.4 / §3: the new row is concatenated on the position axis).
//
// One workgroup per sequence reads lens[s] once. Its threads split the g new
// K rows and g new V rows into UNIT-byte pieces, load every piece they own
// before storing any (so the copy costs one memory round trip, not one per
// row), and write them to slot lens[s]. Only after a barrier does one thread
// write lens[s] + 1, so every thread used the old length. A length outside
// [0, cap) leaves the sequence untouched. With a paged cache (p.pg.table set)
// the slot is row lens[s] mod B of the block the table names for lens[s].
// With n_tok > 1 tokens per sequence (k_new [b][n_tok][g][d]), token r goes
// to position lens[s] + r and the length grows by n_tok (all of them must
// fit below cap, else the sequence is left untouched).
#include "gqa_internal.hpp"

namespace gqa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ size_t slot_row(const AppendParams& p, int s, int j, int pos) {
  return p.pg.table ? kv_row<true, false>(p.pg, p.g, p.cap, s, j, pos) : kv_row<false, false>(p.pg, p.g, p.cap, s, j, pos);
}

template <typename UNIT, int PER_THREAD>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p, int esize) {
  const int s = blockIdx.x;
  __shared__ int s_pos;
  if (threadIdx.x == 0) s_pos = p.lens[s];
  __syncthreads();
  const int pos = s_pos;
  if (pos < 0 || pos > p.cap - p.n_tok) return;  // precondition violated: change nothing
  const int ku = p.d_k * esize / int(sizeof(UNIT));  // units per K row
  const int vu = p.d_v * esize / int(sizeof(UNIT));
  const int kall = p.n_tok * p.g * ku;  // K units of all the sequence's new tokens
  const int total = kall + p.n_tok * p.g * vu;
  const UNIT* kn = static_cast<const UNIT*>(p.k_new) + size_t(s) * kall;
  const UNIT* vn = static_cast<const UNIT*>(p.v_new) + size_t(s) * p.n_tok * p.g * vu;
  UNIT* kc = static_cast<UNIT*>(p.k_cache);
  UNIT* vc = static_cast<UNIT*>(p.v_cache);
  for (int base = 0; base < total; base += PER_THREAD * blockDim.x) {
    UNIT val[PER_THREAD] = {};
    UNIT* dst[PER_THREAD];
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r) {
      const int c = base + r * blockDim.x + threadIdx.x;
      dst[r] = nullptr;
      if (c < total) {
        if (c < kall) {
          const int row = c / ku, x = c - row * ku;  // row = token * g + head
          const int tok = row / p.g, j = row - tok * p.g;
          val[r] = kn[c];
          dst[r] = kc + slot_row(p, s, j, pos + tok) * ku + x;
        } else {
          const int cv = c - kall;
          const int row = cv / vu, x = cv - row * vu;
          const int tok = row / p.g, j = row - tok * p.g;
          val[r] = vn[cv];
          dst[r] = vc + slot_row(p, s, j, pos + tok) * vu + x;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r)
      if (dst[r]) *dst[r] = val[r];
  }
  __syncthreads();
  if (threadIdx.x == 0) p.lens[s] = pos + p.n_tok;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

}  // namespace

hipError_t launch_append(const AppendParams& p, int b, int dtype, hipStream_t stream) {
  const int esize = dtype == 0 ? 4 : 2;
  const size_t kb = size_t(p.d_k) * esize, vb = size_t(p.d_v) * esize;
  auto fits = [&](size_t a) {
    return kb % a == 0 && vb % a == 0 && aligned(p.k_cache, a) && aligned(p.v_cache, a) &&
           aligned(p.k_new, a) && aligned(p.v_new, a);
  };
  const size_t row_units16 = size_t(p.n_tok) * p.g * (kb + vb) / 16;
  int threads = int((row_units16 + 3) / 4);
  threads = threads < 64 ? 64 : (threads > 256 ? 256 : ((threads + 63) / 64) * 64);
  if (fits(16)) {
    hipLaunchKernelGGL((kv_append_kernel<u32x4, 4>), dim3(b), dim3(threads), 0, stream, p, esize);
  } else if (fits(4)) {
    hipLaunchKernelGGL((kv_append_kernel<uint32_t, 4>), dim3(b), dim3(256), 0, stream, p, esize);
  } else {
    hipLaunchKernelGGL((kv_append_kernel<uint16_t, 4>), dim3(b), dim3(256), 0, stream, p, esize);
  }
  return hipGetLastError();
}

}  // namespace gqa
