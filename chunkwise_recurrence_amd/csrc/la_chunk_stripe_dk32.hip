// Instantiations of the stripe kernel for d_k = 32.
#include "la_chunk_stripe.h"

namespace la {
hipError_t launch_chunk_stripe_dk32(const ChunkArgs& a, bool state_only, hipStream_t s) {
  return stripe::dispatch_cat<32>(a, state_only, s);
}
}  // namespace la
