// la_delta.hip -- the delta rule (DeltaNet; with a scalar decay a_t, Gated
// DeltaNet), chunkwise, fp32 arithmetic.
//
// Per head ("Linear / Sparse Attention - minimal runnable implementation",
// delta_rule_recurrent, stored transposed as a d_k x d_v state; the tutorial's
// sections 5.1-5.2, Q15 and Q17 for the gate):
//
//   S_t = a_t (S_{t-1} - beta_t k_t (k_t^T S_{t-1})) + beta_t k_t v_t^T,   o_t = q_t^T S_t
//
// The tutorial's section 5.3 and Q23 say the chunk's product of erase factors
// goes into a compact WY form so that a chunk is matmuls; the steps used here
// come from unrolling the recurrence over one chunk.  With b the in-chunk
// inclusive prefix of log a and G[i,j] = e^{b_i - b_j}, the chunk's
// pseudo-values u_t = beta_t (v_t - a_t S_{t-1}^T k_t) solve a unit
// lower-triangular system, so with T = (I + diag(beta) (tril(K K^T, -1) o G))^-1
//
//   W  = T diag(beta e^b) K,   U0 = T diag(beta) V        (no state: every chunk at once)
//   U  = U0 - W S_c
//   O_c = diag(e^b) Q S_c + ((Q K^T) o tril(G)) U
//   S_{c+1} = e^{b_last} S_c + (diag(e^{b_last - b}) K)^T U
//
// Two kernels: delta_prep_kernel (one workgroup per head and chunk) solves
// each chunk's system by forward substitution and writes W and U0 to the
// workspace in fp32; delta_chunk_kernel (one workgroup per head and 32 value
// columns -- the columns of S are independent under this update) walks the
// chunks in order with its part of S in LDS.  Both keep their tiles in LDS
// as fp32 and use plain FMA.
#include "la_device.h"

namespace la {
namespace {

constexpr int kDeltaTile = 32;  // value columns per workgroup of the chunk pass

template <bool BF16>
__device__ __forceinline__ float ld(const void* p, size_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}
template <bool BF16>
__device__ __forceinline__ void st(void* p, size_t i, float x) {
  if constexpr (BF16) static_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16(x);
  else static_cast<float*>(p)[i] = x;
}

// In-chunk inclusive prefix b of log a over tokens t0 .. t0 + n - 1 of head
// (bh, h), into sb[0..n).  One thread; n <= kDeltaMaxC.
__device__ void chunk_log_prefix(const DeltaArgs& a, int bh, int h, int t0, int n, float* sb) {
  const float lg = a.decay_kind == kDecayHead ? logf(a.decay[h]) : 0.0f;
  const float* dt = (a.decay_kind == kDecayLog || a.decay_kind == kDecayGate)
                        ? a.decay + (size_t)bh * a.L : nullptr;
  float b = 0.0f;
  for (int i = 0; i < n; ++i) {
    if (a.decay_kind == kDecayHead) b += lg;
    else if (dt) b += token_log_decay(a.decay_kind, dt[t0 + i]);
    sb[i] = b;
  }
}

template <bool BF16, int DK>
__global__ __launch_bounds__(256) void delta_prep_kernel(const DeltaArgs a) {
  constexpr int KP = DK + 1;  // padded row stride (fp32 words)
  const int tid = threadIdx.x;
  const int L = a.L, C = a.C, DV = a.DV;
  const int nch = (L + C - 1) / C;
  const int bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int h = bh % a.H;
  const int t0 = c * C, n = min(C, L - t0);

  __shared__ float sK[kDeltaMaxC * KP];
  __shared__ float sV[kDeltaMaxC * (128 + 1)];
  __shared__ float sN[kDeltaMaxC][kDeltaMaxC + 1];
  __shared__ float sT[kDeltaMaxC][kDeltaMaxC + 1];
  __shared__ float sb[kDeltaMaxC], sbeta[kDeltaMaxC];
  const int VP = DV + 1;

  const size_t rowk = (size_t)bh * L + t0;
  for (int idx = tid; idx < n * DK; idx += 256)
    sK[(idx / DK) * KP + idx % DK] = ld<BF16>(a.k, rowk * DK + idx);
  for (int idx = tid; idx < n * DV; idx += 256)
    sV[(idx / DV) * VP + idx % DV] = ld<BF16>(a.v, rowk * DV + idx);
  if (tid < n) sbeta[tid] = a.beta[rowk + tid];
  if (tid == 0) chunk_log_prefix(a, bh, h, t0, n, sb);
  __syncthreads();

  // N[i][j] = beta_i (k_i . k_j) e^{b_i - b_j} below the diagonal
  for (int idx = tid; idx < n * n; idx += 256) {
    const int i = idx / n, j = idx % n;
    float x = 0.0f;
    if (j < i) {
      float dot = 0.0f;
      for (int d = 0; d < DK; ++d) dot = fmaf(sK[i * KP + d], sK[j * KP + d], dot);
      x = sbeta[i] * dot * expf(sb[i] - sb[j]);
    }
    sN[i][j] = x;
  }
  __syncthreads();
  // T = (I + N)^-1 by rows: T[i][j] = [i == j] - sum_{j <= m < i} N[i][m] T[m][j]
  for (int i = 0; i < n; ++i) {
    if (tid < n) {
      const int j = tid;
      float x = j == i ? 1.0f : 0.0f;
      if (j < i) {
        float s = 0.0f;
        for (int m = j; m < i; ++m) s = fmaf(sN[i][m], sT[m][j], s);
        x = -s;
      }
      sT[i][j] = x;
    }
    __syncthreads();
  }
  // W = T diag(beta e^b) K, U0 = T diag(beta) V  (T is lower triangular)
  float* wW = a.ws_W + rowk * DK;
  float* wU = a.ws_U + rowk * DV;
  for (int idx = tid; idx < n * DK; idx += 256) {
    const int i = idx / DK, d = idx % DK;
    float s = 0.0f;
    for (int m = 0; m <= i; ++m) s = fmaf(sT[i][m] * sbeta[m] * expf(sb[m]), sK[m * KP + d], s);
    wW[idx] = s;
  }
  for (int idx = tid; idx < n * DV; idx += 256) {
    const int i = idx / DV, cc = idx % DV;
    float s = 0.0f;
    for (int m = 0; m <= i; ++m) s = fmaf(sT[i][m] * sbeta[m], sV[m * VP + cc], s);
    wU[idx] = s;
  }
}

template <bool BF16, int DK>
__global__ __launch_bounds__(256) void delta_chunk_kernel(const DeltaArgs a) {
  constexpr int KP = DK + 1;
  constexpr int TV = kDeltaTile;
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / a.n_v, vt = blockIdx.x % a.n_v;
  const int h = bh % a.H;
  const int L = a.L, C = a.C, DV = a.DV;
  const int tv = min(TV, DV);
  const int dv0 = vt * tv;

  __shared__ float sQ[kDeltaMaxC * KP], sK[kDeltaMaxC * KP], sW[kDeltaMaxC * KP];
  __shared__ float sU[kDeltaMaxC][TV + 1];
  __shared__ float sS[DK][TV + 1];
  __shared__ float sP[kDeltaMaxC][kDeltaMaxC + 1];
  __shared__ float sb[kDeltaMaxC];

  for (int idx = tid; idx < DK * tv; idx += 256) {
    const int d = idx / tv, cc = idx % tv;
    sS[d][cc] = a.state ? a.state[((size_t)bh * DK + d) * DV + dv0 + cc] : 0.0f;
  }
  for (int t0 = 0; t0 < L; t0 += C) {
    const int n = min(C, L - t0);
    const size_t row = (size_t)bh * L + t0;
    __syncthreads();  // the previous chunk is done with every tile
    for (int idx = tid; idx < n * DK; idx += 256) {
      const int i = idx / DK, d = idx % DK;
      sQ[i * KP + d] = ld<BF16>(a.q, row * DK + idx);
      sK[i * KP + d] = ld<BF16>(a.k, row * DK + idx);
      sW[i * KP + d] = a.ws_W[row * DK + idx];
    }
    for (int idx = tid; idx < n * tv; idx += 256) {
      const int i = idx / tv, cc = idx % tv;
      sU[i][cc] = a.ws_U[(row + i) * DV + dv0 + cc];
    }
    if (tid == 0) chunk_log_prefix(a, bh, h, t0, n, sb);
    __syncthreads();
    // U = U0 - W S (each thread its own elements), scores P = (Q K^T) o tril(G)
    for (int idx = tid; idx < n * tv; idx += 256) {
      const int i = idx / tv, cc = idx % tv;
      float s = sU[i][cc];
      for (int d = 0; d < DK; ++d) s = fmaf(-sW[i * KP + d], sS[d][cc], s);
      sU[i][cc] = s;
    }
    for (int idx = tid; idx < n * n; idx += 256) {
      const int i = idx / n, j = idx % n;
      float p = 0.0f;
      if (j <= i) {
        for (int d = 0; d < DK; ++d) p = fmaf(sQ[i * KP + d], sK[j * KP + d], p);
        p *= expf(sb[i] - sb[j]);
      }
      sP[i][j] = p;
    }
    __syncthreads();
    // O = diag(e^b) Q S + P U
    for (int idx = tid; idx < n * tv; idx += 256) {
      const int i = idx / tv, cc = idx % tv;
      float inter = 0.0f;
      for (int d = 0; d < DK; ++d) inter = fmaf(sQ[i * KP + d], sS[d][cc], inter);
      float intra = 0.0f;
      for (int j = 0; j <= i; ++j) intra = fmaf(sP[i][j], sU[j][cc], intra);
      st<BF16>(a.out, (row + i) * DV + dv0 + cc, expf(sb[i]) * inter + intra);
    }
    __syncthreads();
    // S = e^{b_last} S + (diag(e^{b_last - b}) K)^T U
    const float bL = sb[n - 1];
    for (int idx = tid; idx < DK * tv; idx += 256) {
      const int d = idx / tv, cc = idx % tv;
      float s = 0.0f;
      for (int j = 0; j < n; ++j) s = fmaf(expf(bL - sb[j]) * sK[j * KP + d], sU[j][cc], s);
      sS[d][cc] = fmaf(expf(bL), sS[d][cc], s);
    }
  }
  __syncthreads();
  if (a.state) {
    for (int idx = tid; idx < DK * tv; idx += 256) {
      const int d = idx / tv, cc = idx % tv;
      a.state[((size_t)bh * DK + d) * DV + dv0 + cc] = sS[d][cc];
    }
  }
}

template <bool BF16>
hipError_t launch_dk(const DeltaArgs& a, hipStream_t s) {
  const int nch = (a.L + a.C - 1) / a.C;
  const dim3 gp(a.B * a.H * nch), gc(a.B * a.H * a.n_v), blk(256);
  switch (a.DK) {
#define LA_DK(D)                                                                  \
  case D:                                                                         \
    hipLaunchKernelGGL((delta_prep_kernel<BF16, D>), gp, blk, 0, s, a);           \
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;            \
    hipLaunchKernelGGL((delta_chunk_kernel<BF16, D>), gc, blk, 0, s, a);          \
    return hipGetLastError();
    LA_DK(16)
    LA_DK(32)
    LA_DK(64)
    LA_DK(128)
#undef LA_DK
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_delta(const DeltaArgs& a, hipStream_t s) {
  DeltaArgs b = a;
  const int tv = a.DV < kDeltaTile ? a.DV : kDeltaTile;
  b.n_v = a.DV / tv;
  return a.dtype == kBF16 ? launch_dk<true>(b, s) : launch_dk<false>(b, s);
}

}  // namespace la
