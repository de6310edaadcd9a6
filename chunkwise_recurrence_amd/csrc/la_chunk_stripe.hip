// Dispatch of the stripe kernel (la_chunk_stripe.h) by key dimension, and the
// shapes it supports.
#include "la_chunk_stripe.h"

namespace la {

bool chunk_stripe_supported(int DK, int TVW, int KH, int C, bool channel) {
  if (DK != 32 && DK != 64 && DK != 128) return false;
  if (TVW != 32 && TVW != 64 && TVW != 128) return false;
  if (C != 32 && C != 64 && C != 128) return false;
  if (KH != 1 && !(KH == 2 && DK >= 64)) return false;
  switch (DK) {
    case 32: return stripe::fits_of<32>(TVW, KH, C, channel);
    case 64: return stripe::fits_of<64>(TVW, KH, C, channel);
    default: return stripe::fits_of<128>(TVW, KH, C, channel);
  }
}

hipError_t launch_chunk_stripe(const ChunkArgs& a, bool state_only, hipStream_t s) {
  const int cat = a.decay_kind == kDecayNone      ? stripe::kCatNone
                  : a.decay_kind == kDecayHead    ? stripe::kCatHead
                  : a.decay_kind == kDecayChannel ? stripe::kCatChannel
                                                  : stripe::kCatToken;
#define LA_CASE(DK)                                                       \
  case DK:                                                                \
    return cat == 0 ? launch_chunk_stripe_dk##DK##_c0(a, state_only, s)   \
           : cat == 1 ? launch_chunk_stripe_dk##DK##_c1(a, state_only, s) \
           : cat == 3 ? launch_chunk_stripe_dk##DK##_c3(a, state_only, s) \
                      : launch_chunk_stripe_dk##DK##_c2(a, state_only, s);
  switch (a.DK) {
    LA_CASE(32)
    LA_CASE(64)
    LA_CASE(128)
  }
#undef LA_CASE
  return hipErrorInvalidValue;
}

}  // namespace la
