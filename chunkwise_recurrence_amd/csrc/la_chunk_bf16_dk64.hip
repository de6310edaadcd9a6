// la_chunk_bf16_dk64.hip -- bf16 chunkwise kernels with d_k = 64 (every value tile and chunk size).
#include "la_chunk_bf16.h"

namespace la {

hipError_t launch_chunk_bf16_dk64(const ChunkArgs& a, bool state_only, hipStream_t s) {
  return bf16k::dispatch_cat<64>(a, state_only, s);
}

}  // namespace la
