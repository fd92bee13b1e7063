// Vector-ALU decode attention over paged K/V pools: the PAGED instances of
// the kernel in decode_vector_kernel.hpp (one block-table lookup per
// 32-position tile; see the cache layouts in gqa_internal.hpp).
#include "decode_vector_kernel.hpp"

namespace gqa {

hipError_t launch_decode_vector_paged(const DecodeParams& p, int dtype, hipStream_t stream) {
  return launch_vector<true>(p, dtype, stream);
}

int vector_occupancy_paged(int dtype, int d, int heads_per_block, bool fused) {
  return vector_occupancy<true>(dtype, d, heads_per_block, fused);
}

}  // namespace gqa
