// Vector-ALU decode attention for several new tokens per sequence over paged
// caches: the PAGED and CAUSAL instances of the kernel in
// decode_vector_kernel.hpp (block-table addressing as in the paged one-token
// call, virtual heads and causal limits as in the contiguous multi-token one).
#include "decode_vector_kernel.hpp"

namespace gqa {

hipError_t launch_decode_vector_multi_paged(const DecodeParams& p, int dtype, hipStream_t stream) {
  return launch_vector<true, true>(p, dtype, stream);
}

int vector_occupancy_multi_paged(int dtype, int d, int heads_per_block) {
  return vector_occupancy<true, true>(dtype, d, heads_per_block, false);
}

}  // namespace gqa
