// la_chunk_f32.hip -- chunkwise causal linear attention with fp32 inputs and
// fp32 arithmetic throughout (no bf16 rounding anywhere).
//
// Same chunkwise form as the bf16 kernel (per chunk: inter-chunk term
// diag(e^b) Q_c S_c, intra-chunk term ((Q_c K_c^T) o D_c) V_c, then
// S <- e^{b_last} S + (diag(e^{b_last - b}) K_c)^T V_c), written for
// exactness rather than speed: plain fp32 FMA, the decayed score block and the
// state tile in LDS, q and k read through the caches with phi applied on the
// fly.  One workgroup per (head, 32-column value tile), chunks in sequence.
// It serves small fp32 problems such as the 300 x 16 demo.  The normalised
// form also carries z (z <- e^{b_last} z + sum_j e^{b_last - b_j} phi(k_j)) and
// divides each output row by e^{b_i} phi(q_i).z + sum_{j<=i} P[i][j].
//
// The per-channel gate (the tutorial's section 2.4) makes b a matrix b[t][d]
// of in-chunk prefix sums per key channel; every e^{b...} factor above then
// moves inside the sum over d: P[i][j] = sum_d q_id k_jd e^{b_id - b_jd},
// the inter term is sum_d q_id e^{b_id} S[d][:], and row d of S (entry d of z)
// decays by e^{b_{last,d}}.
#include "la_device.h"

namespace la {
namespace {

constexpr int kTileF32 = 32;   // value columns per workgroup
constexpr int kMaxC = 128;

__device__ __forceinline__ float phi_f32(bool elu, float x) {
  return elu ? feature_elu1_accurate(x) : x;
}

__global__ __launch_bounds__(256) void chunk_f32_kernel(const ChunkArgs a) {
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / a.n_v, vt = blockIdx.x % a.n_v;
  const int h = bh % a.H;
  const int L = a.L, DK = a.DK, DV = a.DV, C = a.C;
  const int tv = min(kTileF32, DV);
  const int dv0 = vt * tv;
  const bool elu = a.phi == kPhiElu1;
  const int kind = a.decay_kind;

  __shared__ float sP[kMaxC * kMaxC];
  __shared__ float sS[128 * kTileF32];
  __shared__ float sB[kMaxC];
  __shared__ float sZ[128], sDen[kMaxC];
  __shared__ float sBc[kMaxC * 128];  // per-channel prefixes b[t][d]
  const bool norm = a.norm != 0;
  const bool chan = kind == kDecayChannel;

  const float* qh = static_cast<const float*>(a.q) + (size_t)bh * L * DK;
  const float* kh = static_cast<const float*>(a.k) + (size_t)bh * L * DK;
  const float* vh = static_cast<const float*>(a.v) + (size_t)bh * L * DV + dv0;
  float* oh = static_cast<float*>(a.out) + (size_t)bh * L * DV + dv0;
  const float* dtok = (kind == kDecayLog || kind == kDecayGate) ? a.decay + (size_t)bh * L : nullptr;
  const float lg = (kind == kDecayHead) ? logf(a.decay[h]) : 0.0f;
  const float* dch = chan ? a.decay + (size_t)bh * L * DK : nullptr;

  for (int i = tid; i < DK * tv; i += 256) {
    const int d = i / tv, v = i % tv;
    sS[i] = a.s0 ? a.s0[((size_t)bh * DK + d) * DV + dv0 + v] : 0.0f;
  }
  if (norm)
    for (int d = tid; d < DK; d += 256) sZ[d] = a.z0 ? a.z0[(size_t)bh * DK + d] : 0.0f;

  for (int t0 = 0; t0 < L; t0 += C) {
    const int n = min(C, L - t0);
    __syncthreads();  // previous chunk's readers of sB / sP are done
    if (tid == 0) {
      float b = 0.0f;
      for (int i = 0; i < n; ++i) {
        if (kind == kDecayHead) b += lg;
        else if (dtok) b += token_log_decay(kind, dtok[t0 + i]);
        sB[i] = b;
      }
    }
    if (chan && tid < DK) {
      float b = 0.0f;
      for (int i = 0; i < n; ++i) {
        b += clamp_log_decay(dch[(size_t)(t0 + i) * DK + tid]);
        sBc[i * DK + tid] = b;
      }
    }
    __syncthreads();
    const float bL = sB[n - 1];
    // decayed scores P[i][j] = (phi(q_i).phi(k_j)) e^{b_i - b_j}, j <= i
    for (int idx = tid; idx < n * n; idx += 256) {
      const int i = idx / n, j = idx % n;
      float p = 0.0f;
      if (j <= i) {
        const float* qi = qh + (size_t)(t0 + i) * DK;
        const float* kj = kh + (size_t)(t0 + j) * DK;
        if (chan) {
          for (int d = 0; d < DK; ++d)
            p = fmaf(phi_f32(elu, qi[d]) * expf(sBc[i * DK + d] - sBc[j * DK + d]),
                     phi_f32(elu, kj[d]), p);
        } else {
          for (int d = 0; d < DK; ++d) p = fmaf(phi_f32(elu, qi[d]), phi_f32(elu, kj[d]), p);
          p *= expf(sB[i] - sB[j]);
        }
      }
      sP[i * kMaxC + j] = p;
    }
    __syncthreads();
    // normalised form: den_i = e^{b_i} phi(q_i).z + sum_{j<=i} P[i][j]
    if (norm) {
      for (int i = tid; i < n; i += 256) {
        const float* qi = qh + (size_t)(t0 + i) * DK;
        float dz = 0.0f, ds = 0.0f;
        if (chan) {
          for (int d = 0; d < DK; ++d)
            dz = fmaf(phi_f32(elu, qi[d]) * expf(sBc[i * DK + d]), sZ[d], dz);
        } else {
          for (int d = 0; d < DK; ++d) dz = fmaf(phi_f32(elu, qi[d]), sZ[d], dz);
          dz *= expf(sB[i]);
        }
        for (int j = 0; j <= i; ++j) ds += sP[i * kMaxC + j];
        sDen[i] = dz + ds;
      }
      __syncthreads();
    }
    // o_i = e^{b_i} phi(q_i)^T S + sum_{j<=i} P[i][j] v_j
    for (int idx = tid; idx < n * tv; idx += 256) {
      const int i = idx / tv, v = idx % tv;
      const float* qi = qh + (size_t)(t0 + i) * DK;
      float inter = 0.0f;
      if (chan) {
        for (int d = 0; d < DK; ++d)
          inter = fmaf(phi_f32(elu, qi[d]) * expf(sBc[i * DK + d]), sS[d * tv + v], inter);
      } else {
        for (int d = 0; d < DK; ++d) inter = fmaf(phi_f32(elu, qi[d]), sS[d * tv + v], inter);
        inter *= expf(sB[i]);
      }
      float intra = 0.0f;
      for (int j = 0; j <= i; ++j) intra = fmaf(sP[i * kMaxC + j], vh[(size_t)(t0 + j) * DV + v], intra);
      const float o = inter + intra;
      oh[(size_t)(t0 + i) * DV + v] = norm ? o / sDen[i] : o;
    }
    __syncthreads();
    // S <- e^{b_last} S + sum_j e^{b_last - b_j} phi(k_j) v_j^T
    for (int idx = tid; idx < DK * tv; idx += 256) {
      const int d = idx / tv, v = idx % tv;
      const float bLd = chan ? sBc[(n - 1) * DK + d] : bL;
      float acc = 0.0f;
      for (int j = 0; j < n; ++j) {
        const float bj = chan ? sBc[j * DK + d] : sB[j];
        acc = fmaf(expf(bLd - bj) * phi_f32(elu, kh[(size_t)(t0 + j) * DK + d]),
                   vh[(size_t)(t0 + j) * DV + v], acc);
      }
      sS[idx] = expf(bLd) * sS[idx] + acc;
    }
    if (norm) {
      for (int d = tid; d < DK; d += 256) {
        const float bLd = chan ? sBc[(n - 1) * DK + d] : bL;
        float acc = 0.0f;
        for (int j = 0; j < n; ++j) {
          const float bj = chan ? sBc[j * DK + d] : sB[j];
          acc = fmaf(expf(bLd - bj), phi_f32(elu, kh[(size_t)(t0 + j) * DK + d]), acc);
        }
        sZ[d] = expf(bLd) * sZ[d] + acc;
      }
    }
  }
  __syncthreads();
  if (a.state) {
    for (int i = tid; i < DK * tv; i += 256) {
      const int d = i / tv, v = i % tv;
      a.state[((size_t)bh * DK + d) * DV + dv0 + v] = sS[i];
    }
  }
  if (norm && a.zstate && vt == 0)
    for (int d = tid; d < DK; d += 256) a.zstate[(size_t)bh * DK + d] = sZ[d];
}

}  // namespace

hipError_t launch_chunk_f32(const ChunkArgs& a, hipStream_t s) {
  ChunkArgs b = a;
  const int tv = a.DV < kTileF32 ? a.DV : kTileF32;
  b.n_v = a.DV / tv;
  b.tv = tv;
  const dim3 grid(a.B * a.H * b.n_v), block(256);
  hipLaunchKernelGGL(chunk_f32_kernel, grid, block, 0, s, b);
  return hipGetLastError();
}

}  // namespace la
