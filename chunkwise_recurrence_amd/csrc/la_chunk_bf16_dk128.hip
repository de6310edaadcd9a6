// la_chunk_bf16_dk128.hip -- bf16 chunkwise kernels with d_k = 128 (every value tile and chunk size).
#include "la_chunk_bf16.h"

namespace la {

hipError_t launch_chunk_bf16_dk128(const ChunkArgs& a, bool state_only, hipStream_t s) {
  return bf16k::dispatch_cat<128>(a, state_only, s);
}

}  // namespace la
