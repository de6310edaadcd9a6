// Instantiations of the stripe kernel for d_k = 128, decay category 3
// (0 none, 1 per head, 2 per token, 3 per key channel); one file each so they compile in parallel.
#include "la_chunk_stripe.h"

namespace la {
hipError_t launch_chunk_stripe_dk128_c3(const ChunkArgs& a, bool state_only, hipStream_t s) {
  return stripe::dispatch_w<128, 3>(a, state_only, s);
}
}  // namespace la
