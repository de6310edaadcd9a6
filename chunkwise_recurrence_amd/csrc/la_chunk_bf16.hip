// la_chunk_bf16.hip -- dispatch of the bf16 chunkwise kernels by key dimension.
#include "la_chunk_bf16.h"

namespace la {
namespace {

// b_t = log2(e) * (sum of log a over the tokens of t's chunk up to and
// including t), for the token-dependent decays (the kernels work in log2
// units so that every decay factor is one v_exp_f32).  One wave takes
// kPrefixChunks consecutive chunks, their loads issued together; per chunk,
// one wave64 inclusive scan (two tokens per lane, chunks of at most 128
// tokens).  The gate's softplus takes the hardware exp2 / log2
// (token_log_decay_fast): the library's expf and log1pf made up most of the
// pass's time.
constexpr int kPrefixChunks = 4;
__global__ __launch_bounds__(256) void decay_prefix_kernel(const ChunkArgs a, int total_chunks) {
  const int lane = threadIdx.x & 63;
  const int g0 = (blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * kPrefixChunks;
  const int nchunks = (a.L + a.C - 1) / a.C;
  const int i0 = 2 * lane, i1 = 2 * lane + 1;
  constexpr float kLog2e = 1.4426950408889634f;
  float r0[kPrefixChunks], r1[kPrefixChunks];
#pragma unroll
  for (int k = 0; k < kPrefixChunks; ++k) {
    const int gid = g0 + k;
    const int bh = gid / nchunks, t0 = (gid % nchunks) * a.C;
    const float* in = a.decay + (size_t)bh * a.L;
    const bool ok = gid < total_chunks;
    r0[k] = ok && i0 < a.C && t0 + i0 < a.L ? in[t0 + i0] : 0.0f;
    r1[k] = ok && i1 < a.C && t0 + i1 < a.L ? in[t0 + i1] : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < kPrefixChunks; ++k) {
    const int gid = g0 + k;
    if (gid >= total_chunks) break;
    const int bh = gid / nchunks, t0 = (gid % nchunks) * a.C;
    float* out = a.ws_b + (size_t)bh * a.L;
    const bool v0 = i0 < a.C && t0 + i0 < a.L, v1 = i1 < a.C && t0 + i1 < a.L;
    const float x0 = v0 ? token_log_decay_fast(a.decay_kind, r0[k]) * kLog2e : 0.0f;
    const float x1 = v1 ? token_log_decay_fast(a.decay_kind, r1[k]) * kLog2e : 0.0f;
    float s = x0 + x1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(s, off, 64);
      if (lane >= off) s += y;
    }
    if (v0) out[t0 + i0] = s - x1;
    if (v1) out[t0 + i1] = s;
  }
}

}  // namespace

hipError_t launch_decay_prefix(const ChunkArgs& a, hipStream_t s) {
  const int nchunks = (a.L + a.C - 1) / a.C;
  const int total = a.B * a.H * nchunks;
  const int waves = (total + kPrefixChunks - 1) / kPrefixChunks;
  hipLaunchKernelGGL(decay_prefix_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, a, total);
  return hipGetLastError();
}

bool chunk_bf16_supported(int DK, int TV, int NG, int C) {
  if (C != 16 && C != 32 && C != 64 && C != 128) return false;
  if (TV != 16 && TV != 32 && TV != 64) return false;
  if (NG != 1 && NG != 2) return false;
  size_t lds = 0;
  switch (DK) {
    case 16: lds = bf16k::lds_tv<16>(TV, NG, C); break;
    case 32: lds = bf16k::lds_tv<32>(TV, NG, C); break;
    case 64: lds = bf16k::lds_tv<64>(TV, NG, C); break;
    case 128: lds = bf16k::lds_tv<128>(TV, NG, C); break;
    default: return false;
  }
  return lds <= bf16k::kMaxLds;
}

hipError_t launch_chunk_bf16(const ChunkArgs& a, bool state_only, hipStream_t s) {
  switch (a.DK) {
    case 16: return launch_chunk_bf16_dk16(a, state_only, s);
    case 32: return launch_chunk_bf16_dk32(a, state_only, s);
    case 64: return launch_chunk_bf16_dk64(a, state_only, s);
    case 128: return launch_chunk_bf16_dk128(a, state_only, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace la
