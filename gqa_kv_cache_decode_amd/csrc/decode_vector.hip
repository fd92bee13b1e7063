// Vector-ALU decode attention: the contiguous-cache instances of the kernel
// in decode_vector_kernel.hpp, and the launch and occupancy entry points of
// every variant (the paged instances are in decode_vector_paged.hip, the
// multi-token ones in decode_vector_multi.hip and, over paged caches,
// decode_vector_multi_paged.hip).
#include <atomic>

#include "decode_vector_kernel.hpp"

namespace gqa {

int vector_waves(int dtype, int d, int heads_per_block) {
  const int esize = dtype == 0 ? 4 : 2;
  return (heads_per_block <= 4 && heads_per_block * d * esize <= 512) ? 8 : 4;
}

// Kept once per process like matrix_workgroups_per_cu (relaxed atomics).
int vector_workgroups_per_cu(int dtype, int d, int heads_per_block, bool fused, bool paged, bool causal) {
  // kind: 0 one-token, 1 fused step, 2 paged, 3 paged fused step, 4 multi-token, 5 paged multi-token
  static std::atomic<int> cached[6][2][5][4] = {};
  const int ti = dtype == 0 ? 0 : 1;
  const int di = d == 16 ? 0 : d == 32 ? 1 : d == 64 ? 2 : d == 128 ? 3 : 4;
  const int hi = heads_per_block == 1 ? 0 : heads_per_block == 2 ? 1 : heads_per_block == 4 ? 2 : 3;
  const int kind = causal ? (paged ? 5 : 4) : (paged ? 2 : 0) + (fused ? 1 : 0);
  std::atomic<int>& c = cached[kind][ti][di][hi];
  const int known = c.load(std::memory_order_relaxed);
  if (known > 0) return known;
  const int n = causal ? (paged ? vector_occupancy_multi_paged(dtype, d, heads_per_block)
                                 : vector_occupancy_multi(dtype, d, heads_per_block))
                       : paged ? vector_occupancy_paged(dtype, d, heads_per_block, fused)
                               : vector_occupancy<false>(dtype, d, heads_per_block, fused);
  if (n > 0) c.store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_decode_vector(const DecodeParams& p, int dtype, hipStream_t stream) {
  if (p.n_tok > 1)
    return p.pg.table ? launch_decode_vector_multi_paged(p, dtype, stream) : launch_decode_vector_multi(p, dtype, stream);
  if (p.pg.table) return launch_decode_vector_paged(p, dtype, stream);
  return launch_vector<false>(p, dtype, stream);
}

}  // namespace gqa
