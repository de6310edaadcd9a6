// la_device.h -- small device helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_internal.h"

namespace la {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// phi(x) = elu(x) + 1 (alpha = 1): x + 1 for x > 0, e^x otherwise.
// phi = elu + 1 as max(x + 1, e^{-|x|}): since e^x >= 1 + x, the maximum is
// x + 1 for x > 0 (where e^{-x} < 1 < x + 1) and e^x for x <= 0.  Four VALU
// instructions per value (the -|.| is a source modifier of v_exp_f32), no
// compare and select; the same bf16 result as the branch form for every
// bf16 input.
__device__ __forceinline__ float feature_elu1(float x) {
  return fmaxf(x + 1.0f, __builtin_amdgcn_exp2f(-fabsf(x * 1.4426950408889634f)));
}

__device__ __forceinline__ float feature_elu1_accurate(float x) {
  return x > 0.0f ? x + 1.0f : expf(x);
}

// x of the lane D below (row_shr) or above (row_shl) in the same 16-lane row
// (DPP); a lane with none in its row gets 0.  Every lane must be active.
template <int D>
__device__ __forceinline__ float dpp_row_shr(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + D, 0xf, 0xf, false));
}
template <int D>
__device__ __forceinline__ float dpp_row_shl(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x100 + D, 0xf, 0xf, false));
}

// Smallest per-token log decay the kernels work with: ln of the smallest
// normal fp32 (2^-126).  A decay below it, -inf included, is taken as 2^-126:
// every factor that contains it is then below the fp32 normal range, as the
// true one is, and the in-chunk prefix sums stay finite (no inf - inf) and
// small enough (|b| <= 126 C in log2 units) for their differences to keep
// their precision.  NaN is kept.
constexpr float kMinLogDecay = -87.33654475f;
__device__ __forceinline__ float clamp_log_decay(float x) {
  return x < kMinLogDecay ? kMinLogDecay : x;
}

// log a_t for the token-dependent decay kinds (0 for none).
//   log:  the value itself;  gate: -softplus(g) = -(max(g,0) + log1p(e^-|g|)).
__device__ __forceinline__ float token_log_decay(int kind, float x) {
  if (kind == kDecayLog) return clamp_log_decay(x);
  if (kind == kDecayGate) return clamp_log_decay(-(fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)))));
  return 0.0f;
}

// The same from the hardware exp2 / log2 (a few ulp; for the bf16 paths):
// log1p(y) = ln(u) - ((u - 1) - y) / u with u = 1 + y, the second term
// undoing the rounding of u (so log1p(y) = y for tiny y).
__device__ __forceinline__ float token_log_decay_fast(int kind, float x) {
  if (kind == kDecayLog) return clamp_log_decay(x);
  if (kind == kDecayGate) {
    const float y = __builtin_amdgcn_exp2f(-fabsf(x * 1.4426950408889634f));
    const float u = 1.0f + y;
    const float l1p = __builtin_amdgcn_logf(u) * 0.6931471805599453f -
                      ((u - 1.0f) - y) * __builtin_amdgcn_rcpf(u);
    return clamp_log_decay(-(fmaxf(x, 0.0f) + l1p));
  }
  return 0.0f;
}

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Global -> LDS copies: lane l of the wave writes bytes [16 l, 16 l + 16) (or
// [4 l, 4 l + 4)) past dst, which is wave-uniform and goes to M0.  They are
// issued from inline asm on purpose: the compiler tracks copies made with the
// builtin and, unable to tell that the buffers they fill are not the ones read
// or written meanwhile, puts a full vmcnt(0) wait before later LDS accesses,
// which drains the next chunk's prefetch (and the output stores) in the middle
// of every chunk.  Hidden from the compiler, the copies are ordered only by
// the kernels' own counted waits (s_waitcnt vmcnt) and barriers.  They write
// no register, and M0 is restored after each one.
// (The low 32 bits of a generic pointer into LDS are its LDS address.)
__device__ __forceinline__ uint32_t lds_u32(void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)p);
}
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(keep) : "v"(src), "s"(lds_u32(dst)) : "memory");
}
// The same with the non-temporal hint, for data read for the last time.
__device__ __forceinline__ void dma16_nt(const void* src, void* dst) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
      : "=&s"(keep) : "v"(src), "s"(lds_u32(dst)) : "memory");
}
__device__ __forceinline__ void dma4(const void* src, void* dst) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(keep) : "v"(src), "s"(lds_u32(dst)) : "memory");
}

}  // namespace la
