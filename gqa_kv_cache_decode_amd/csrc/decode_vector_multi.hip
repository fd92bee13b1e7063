// Vector-ALU decode attention for several new tokens per sequence: the
// CAUSAL instances of the kernel in decode_vector_kernel.hpp (contiguous
// caches; each KV group's n_tok * G virtual heads taken a head block at a
// time, token r's heads limited to the positions up to itself).
#include "decode_vector_kernel.hpp"

namespace gqa {

hipError_t launch_decode_vector_multi(const DecodeParams& p, int dtype, hipStream_t stream) {
  return launch_vector<false, true>(p, dtype, stream);
}

int vector_occupancy_multi(int dtype, int d, int heads_per_block) {
  return vector_occupancy<false, true>(dtype, d, heads_per_block, false);
}

}  // namespace gqa
