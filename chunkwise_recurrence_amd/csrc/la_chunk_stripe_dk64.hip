// Instantiations of the stripe kernel for d_k = 64.
#include "la_chunk_stripe.h"

namespace la {
hipError_t launch_chunk_stripe_dk64(const ChunkArgs& a, bool state_only, hipStream_t s) {
  return stripe::dispatch_cat<64>(a, state_only, s);
}
}  // namespace la
