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
// Two passes: delta_prep_kernel (one workgroup per head and chunk) solves
// each chunk's system and writes W and U0 (and, on the matrix-core path, the
// chunk's causal scores) to the workspace; then one
// workgroup per head and 32 value columns (the columns of S are independent
// under this update) walks the chunks in order: delta_chunk_mfma_kernel for
// bf16 inputs with C = 64 (bf16 MFMA operands, fp32 accumulation, the state
// in accumulators), delta_chunk_kernel otherwise (fp32 tiles in LDS, plain
// FMA, no bf16 rounding anywhere).
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

// Workgroup barrier for data exchanged through LDS only: this wave's LDS
// accesses complete (lgkmcnt(0)), then s_barrier.  No memory fence, so global
// loads and stores in flight stay in flight (__syncthreads would wait for
// them).  The empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Two fp32 values to packed bf16 (round to nearest even) with the hardware
// conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transpose read of a row-major bf16 LDS tile with a row stride of `stride`
// elements: lane i of each 16-lane group receives column col0 + i of rows
// k0 .. k0 + 7 (two ds_read_b64_tr_b16, each source lane addressing 4 columns
// of one row).  The 8 values are the k-run of an MFMA operand lane.  Every
// lane of the wave must take part.
__device__ __forceinline__ u32x4 lds_tr8(const uint16_t* base, int stride, int k0, int col0,
                                         int l16) {
  const int j = l16 >> 2, m = l16 & 3;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(base + (k0 + j) * stride + col0 + 4 * m));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(base + (k0 + 4 + j) * stride + col0 + 4 * m));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// log a_t of token t (0 past the sequence)
__device__ __forceinline__ float token_log(const DeltaArgs& a, float lg, const float* dt, int t) {
  if (a.decay_kind == kDecayHead) return lg;
  if (dt) return token_log_decay(a.decay_kind, dt[t]);
  return 0.0f;
}

// Inclusive prefix of log a over the chunk's tokens by wave 0 (C <= 64):
// lane t holds token t0 + t; tokens past the sequence add nothing, so
// sb[t] for t >= n repeats b_last.
__device__ __forceinline__ void chunk_log_prefix_wave(const DeltaArgs& a, int bh, int h, int t0,
                                                      int n, float* sb) {
  const int lane = threadIdx.x & 63;
  const float lg = a.decay_kind == kDecayHead ? logf(a.decay[h]) : 0.0f;
  const float* dt = (a.decay_kind == kDecayLog || a.decay_kind == kDecayGate)
                        ? a.decay + (size_t)bh * a.L + t0 : nullptr;
  float x = lane < n ? token_log(a, lg, dt, lane) : 0.0f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane < a.C) sb[lane] = x;
}

// The same prefix from decay data already in a register: lane t of wave 0
// holds the raw value of token t0 + t (gamma's log for the per-head kind).
// In log2 units (b log2(e)), so that every factor is one v_exp_f32.
__device__ __forceinline__ void chunk_log_prefix_reg(const DeltaArgs& a, float raw, int n, float* sb) {
  const int lane = threadIdx.x & 63;
  constexpr float kLog2e = 1.4426950408889634f;
  float x = 0.0f;
  if (lane < n) {
    if (a.decay_kind == kDecayHead) x = raw * kLog2e;
    else if (a.decay_kind == kDecayLog || a.decay_kind == kDecayGate)
      x = token_log_decay(a.decay_kind, raw) * kLog2e;
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane < a.C) sb[lane] = x;
}

// One workgroup per (head, chunk): T = (I + N)^-1 with
// N = diag(beta) (tril(K K^T, -1) o G) by 16 x 16 blocks (diagonal blocks by
// forward substitution, all at once; then block rows I = 1.. with
// T_IJ = -T_II sum_{J <= M < I} N_IM T_MJ), then W = T diag(beta e^b) K and
// U0 = T diag(beta) V, both in fp32 (the fp32-arithmetic path).
template <bool BF16, int DK>
__global__ __launch_bounds__(256) void delta_prep_kernel(const DeltaArgs a) {
  constexpr int KP = DK + 1;  // padded row stride (fp32 words)
  const int tid = threadIdx.x;
  const int L = a.L, C = a.C, DV = a.DV;
  const int nch = (L + C - 1) / C;
  const int bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int h = bh % a.H;
  const int t0 = c * C, n = min(C, L - t0);
  const int NB = C / 16;  // 16 x 16 blocks per side

  __shared__ float sK[kDeltaMaxC * KP];
  __shared__ float sV[kDeltaMaxC * (128 + 1)];
  __shared__ float sN[kDeltaMaxC][kDeltaMaxC + 1];
  __shared__ float sT[kDeltaMaxC][kDeltaMaxC + 1];
  __shared__ float sX[3 * 16][17];
  __shared__ float sb[kDeltaMaxC], sbeta[kDeltaMaxC];
  const int VP = DV + 1;

  const size_t rowk = (size_t)bh * L + t0;
  for (int idx = tid; idx < n * DK; idx += 256)
    sK[(idx / DK) * KP + idx % DK] = ld<BF16>(a.k, rowk * DK + idx);
  for (int idx = tid; idx < n * DV; idx += 256)
    sV[(idx / DV) * VP + idx % DV] = ld<BF16>(a.v, rowk * DV + idx);
  if (tid < C) sbeta[tid] = tid < n ? a.beta[rowk + tid] : 0.0f;
  if (tid < 64) chunk_log_prefix_wave(a, bh, h, t0, n, sb);
  for (int idx = tid; idx < C * C; idx += 256) sT[idx / C][idx % C] = 0.0f;
  __syncthreads();

  // N[i][j] = beta_i (k_i . k_j) e^{b_i - b_j} below the diagonal (0 past the sequence)
  for (int idx = tid; idx < C * C; idx += 256) {
    const int i = idx / C, j = idx % C;
    float x = 0.0f;
    if (j < i && i < n) {
      float dot = 0.0f;
      for (int d = 0; d < DK; ++d) dot = fmaf(sK[i * KP + d], sK[j * KP + d], dot);
      x = sbeta[i] * dot * expf(sb[i] - sb[j]);
    }
    sN[i][j] = x;
  }
  __syncthreads();
  // diagonal blocks: T[i][j] = [i == j] - sum_{j <= m < i} N[i][m] T[m][j] inside each block
  for (int i = 0; i < 16; ++i) {
    if (tid < 16 * NB) {
      const int q0 = 16 * (tid >> 4), j = tid & 15;
      float x = i == j ? 1.0f : 0.0f;
      if (j < i) {
        float s2 = 0.0f;
        for (int m = j; m < i; ++m) s2 = fmaf(sN[q0 + i][q0 + m], sT[q0 + m][q0 + j], s2);
        x = -s2;
      }
      sT[q0 + i][q0 + j] = x;
    }
    __syncthreads();
  }
  // block rows below: X_J = sum_{J <= M < I} N_IM T_MJ, then T_IJ = -T_II X_J
  for (int I = 1; I < NB; ++I) {
    for (int idx = tid; idx < I * 256; idx += 256) {
      const int J = idx >> 8, r = (idx >> 4) & 15, cc = idx & 15;
      float x = 0.0f;
      for (int m = 16 * J; m < 16 * I; ++m) x = fmaf(sN[16 * I + r][m], sT[m][16 * J + cc], x);
      sX[16 * J + r][cc] = x;
    }
    __syncthreads();
    for (int idx = tid; idx < I * 256; idx += 256) {
      const int J = idx >> 8, r = (idx >> 4) & 15, cc = idx & 15;
      float x = 0.0f;
      for (int m = 0; m < 16; ++m) x = fmaf(sT[16 * I + r][16 * I + m], sX[16 * J + m][cc], x);
      sT[16 * I + r][16 * J + cc] = -x;
    }
    __syncthreads();
  }
  // scale the rows once: K row m by beta_m e^{b_m}, V row m by beta_m
  for (int idx = tid; idx < n * DK; idx += 256) {
    const int m = idx / DK;
    sK[m * KP + idx % DK] *= sbeta[m] * expf(sb[m]);
  }
  for (int idx = tid; idx < n * DV; idx += 256) {
    const int m = idx / DV;
    sV[m * VP + idx % DV] *= sbeta[m];
  }
  __syncthreads();
  // W = T K~, U0 = T V~, four adjacent columns per thread
  for (int idx = tid; idx < n * (DK / 4); idx += 256) {
    const int i = idx / (DK / 4), d0 = 4 * (idx % (DK / 4));
    float x0 = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
    for (int m = 0; m <= i; ++m) {
      const float t = sT[i][m];
      const float* kr = &sK[m * KP + d0];
      x0 = fmaf(t, kr[0], x0);
      x1 = fmaf(t, kr[1], x1);
      x2 = fmaf(t, kr[2], x2);
      x3 = fmaf(t, kr[3], x3);
    }
    *reinterpret_cast<float4*>(a.ws_W + (rowk + i) * DK + d0) = make_float4(x0, x1, x2, x3);
  }
  for (int idx = tid; idx < n * (DV / 4); idx += 256) {
    const int i = idx / (DV / 4), c0 = 4 * (idx % (DV / 4));
    float x0 = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
    for (int m = 0; m <= i; ++m) {
      const float t = sT[i][m];
      const float* vr = &sV[m * VP + c0];
      x0 = fmaf(t, vr[0], x0);
      x1 = fmaf(t, vr[1], x1);
      x2 = fmaf(t, vr[2], x2);
      x3 = fmaf(t, vr[3], x3);
    }
    *reinterpret_cast<float4*>(a.ws_U + (rowk + i) * DV + c0) = make_float4(x0, x1, x2, x3);
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
  __shared__ float sb[kDeltaMaxC], swt[kDeltaMaxC];

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
    // U = U0 - W S (each thread its own elements), scores P = (Q K^T) o tril(G),
    // update weights e^{b_last - b_j}
    if (tid < n) swt[tid] = expf(sb[n - 1] - sb[tid]);
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
      for (int j = 0; j < n; ++j) s = fmaf(swt[j] * sK[j * KP + d], sU[j][cc], s);
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

// The solve pass for bf16 inputs with C = 64 (the MFMA path): one workgroup
// of 4 waves per (head, chunk).
//   * G = K K^T on v_mfma_f32_16x16x32_bf16 (exact products of the bf16
//     inputs, fp32 sums), N = diag(beta) (tril(G, -1) o e^{b_i - b_j}) in LDS.
//   * T = (I + N)^-1, formed in place of N: wave w inverts diagonal block w
//     by forward substitution with its 16 columns in registers (lane j holds
//     column j, no barriers); the blocks below the diagonal follow block row
//     by block row, T_IJ = -T_II sum_{J <= M < I} N_IM T_MJ, on fp32 MFMA.
//   * W = (T diag(beta e^b)) K and U0 = (T diag(beta)) V on MFMA, with the
//     fp32 left factor split into a bf16 high part and a bf16 remainder (two
//     MFMAs, ~16 significant bits; each wave splits its own rows in
//     registers); W and U0 leave as bf16.
//   * the chunk's causal scores (q_i . k_j) e^{b_i - b_j} [j <= i] as bf16
//     rows, computed here once per head and chunk instead of once per value
//     tile in the sequential pass, and the in-chunk prefix b itself (fp32,
//     log2 units), whose gate logarithms and scan would otherwise sit on the
//     sequential pass's chunk-to-chunk chain.
template <int DK>
__global__ __launch_bounds__(256) void delta_prep_mfma_kernel(const DeltaArgs a) {
  constexpr int C = 64, QS = DK + 8, CS = C + 8, KST = DK / 32, NCH = DK / 8;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int L = a.L, DV = a.DV;
  const int nch = (L + C - 1) / C;
  const int bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int h = bh % a.H;
  const int t0 = c * C, n = min(C, L - t0);

  constexpr int VS = 128 + 8;  // row stride of the V tile (d_v <= 128)
  // K until W is formed, then V (which waits in registers until then).  T is
  // formed in place of N (block row by block row: N's blocks of a row are
  // dead once that row of T is known), the X blocks of the inverse sit in
  // the upper triangle, which neither fills, and each wave splits its own
  // rows of the left factor in registers: 34.5 KB at d_k = 128, four
  // workgroups per compute unit
  __shared__ __align__(16) uint16_t sKV[C * (QS > VS ? QS : VS)];
  uint16_t* const sK = sKV;
  uint16_t* const sV = sKV;
  __shared__ float sT[C][C + 1];
  float (*const sN)[C + 1] = sT;
  __shared__ float sb[C], sbeta[C];

  const size_t rowk = (size_t)bh * L + t0;
  const uint16_t* kc = static_cast<const uint16_t*>(a.k) + rowk * DK;
  const uint16_t* vc = static_cast<const uint16_t*>(a.v) + rowk * DV;
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
  // (the query rows past the sequence re-read its last row, unconditionally,
  // and are zeroed where the value is used: a load under a condition makes
  // the compiler wait for it on the spot)
  const int iq = 16 * w + l16;
  u32x4 bq[KST];
  const bool tok = a.decay_kind == kDecayLog || a.decay_kind == kDecayGate;
  float rbeta, rdec = 0.0f;
  // The loads, in the order their data is needed: the K tile (the first
  // barrier publishes it), beta and (wave 0) the decay data of token t0 + lane
  // (stored before that barrier), the query row 16w + l16 as the B operand
  // of the score tiles (used after it), and the V tile (used last; it stays
  // in registers until the LDS buffer it shares with K is free).  Every load
  // is issued before the first LDS store, so the workgroup (one chunk) waits
  // for memory once, and each wait covers only the loads issued before what
  // it waits for.  A whole chunk takes no row checks; the short last chunk of
  // a sequence re-reads its last row and zeroes the rows past it.
  constexpr int PK = C * NCH / 256;   // 16-byte pieces of K per thread
  constexpr int PV = C * 16 / 256;    // ... of V at most (d_v <= 128)
  static_assert(PK >= 1 && C * NCH % 256 == 0, "K tile pieces per thread");
  const int VCH = DV / 8;
  const bool whole_chunk = n == C;
  u32x4 xv[PV];
  auto stage = [&](bool whole) {
    u32x4 xk[PK];
#pragma unroll
    for (int p = 0; p < PK; ++p) {
      const int idx = tid + 256 * p, row = idx / NCH, ch = idx % NCH;
      xk[p] = *reinterpret_cast<const u32x4*>(kc + (size_t)(whole ? row : min(row, n - 1)) * DK + 8 * ch);
    }
    rbeta = a.beta[rowk + min(tid, n - 1)];
    if (w == 0) {
      if (tok) rdec = a.decay[rowk + min(lane, n - 1)];
      else if (a.decay_kind == kDecayHead) rdec = logf(a.decay[h]);
    }
    {
      const uint16_t* qr = static_cast<const uint16_t*>(a.q) + (rowk + min(iq, n - 1)) * DK;
#pragma unroll
      for (int s = 0; s < KST; ++s) bq[s] = *reinterpret_cast<const u32x4*>(qr + 32 * s + 8 * g4);
    }
    // (pieces past a narrower V tile repeat its last piece, load and store)
#pragma unroll
    for (int p = 0; p < PV; ++p) {
      const int idx = min(tid + 256 * p, C * VCH - 1), row = idx / VCH, ch = idx % VCH;
      xv[p] = *reinterpret_cast<const u32x4*>(vc + (size_t)(whole ? row : min(row, n - 1)) * DV + 8 * ch);
    }
#pragma unroll
    for (int p = 0; p < PK; ++p) {
      const int idx = tid + 256 * p, row = idx / NCH, ch = idx % NCH;
      *reinterpret_cast<u32x4*>(&sK[row * QS + 8 * ch]) = (whole || row < n) ? xk[p] : zero4;
    }
  };
  if (n == C) stage(true);
  else stage(false);
  if (tid < C) sbeta[tid] = tid < n ? rbeta : 0.0f;
  lds_barrier();  // the K tile is in LDS

  // The chunk's 20 score tiles: N = K K^T below and on the diagonal (10
  // tiles, operands from the K tile) and the causal scores P = K q (wave w:
  // query rows 16w .. 16w + 15, key tiles 0..w, q in registers).  Their
  // products need no decay factors, so they run before the barrier that
  // publishes the prefix b, which wave 0 forms meanwhile: wave 0 takes only
  // its one P tile, and the N tiles are dealt to waves 1-3 (4, 3, 3; with
  // their 2, 3, 4 P tiles, 6, 6 and 7 tiles each).
  // N tile t (row block, key block): nibble t of these, tiles in row-major
  // order (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ..
  constexpr unsigned long long kNR = 0x3333222110ull, kNJ = 0x3210210100ull;
  const int n_first = w == 0 ? 0 : w == 1 ? 0 : w == 2 ? 4 : 7;
  const int n_count = w == 0 ? 0 : w == 1 ? 4 : 3;
  f32x4 accN[4], accP[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    accN[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (u < n_count) {
      const int R = (int)((kNR >> (4 * (n_first + u))) & 15), J = (int)((kNJ >> (4 * (n_first + u))) & 15);
#pragma unroll
      for (int s = 0; s < KST; ++s) {
        const u32x4 ai = *reinterpret_cast<const u32x4*>(&sK[(16 * R + l16) * QS + 32 * s + 8 * g4]);
        const u32x4 bj = *reinterpret_cast<const u32x4*>(&sK[(16 * J + l16) * QS + 32 * s + 8 * g4]);
        accN[u] = mfma16x16x32(ai, bj, accN[u]);
      }
    }
  }
  const int i_q = iq;
#pragma unroll
  for (int jt = 0; jt < C / 16; ++jt) {
    accP[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (jt <= w) {
#pragma unroll
      for (int s = 0; s < KST; ++s) {
        const u32x4 ak = *reinterpret_cast<const u32x4*>(&sK[(16 * jt + l16) * QS + 32 * s + 8 * g4]);
        accP[jt] = mfma16x16x32(ak, i_q < n ? bq[s] : zero4, accP[jt]);
      }
    }
  }
  if (w == 0) {
    chunk_log_prefix_reg(a, rdec, n, sb);  // log2 units
    // for the sequential pass, which then has no prefix to form on its
    // chunk-to-chunk critical path
    if (lane < n) a.ws_b[rowk + lane] = sb[lane];
  }
  lds_barrier();  // the prefix b is in LDS

  // N[i][j] = beta_i (k_i . k_j) e^{b_i - b_j} for j < i
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (u < n_count) {
      const int R = (int)((kNR >> (4 * (n_first + u))) & 15), J = (int)((kNJ >> (4 * (n_first + u))) & 15);
      const int j = 16 * J + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * R + 4 * g4 + r;
        sN[i][j] = (j < i && i < n) ? sbeta[i] * accN[u][r] * ex2(sb[i] - sb[j]) : 0.0f;
      }
    }
  }
  // P rows for the sequential pass, which then needs no score products of its
  // own: every token column (zeros above the diagonal), bf16
  {
    const int i = i_q;
    uint16_t* po = static_cast<uint16_t*>(a.ws_P) + (rowk + i) * C;
#pragma unroll
    for (int jt = 0; jt < C / 16; ++jt) {
      // register r: token j = 16 jt + 4 g4 + r of query row i
      float pv[4] = {0.f, 0.f, 0.f, 0.f};
      if (jt <= w) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * jt + 4 * g4 + r;
          pv[r] = j <= i ? accP[jt][r] * ex2(sb[i] - sb[j]) : 0.0f;
        }
      }
      if (i < n) *reinterpret_cast<uint2*>(po + 16 * jt + 4 * g4) = make_uint2(cvt2(pv[0], pv[1]), cvt2(pv[2], pv[3]));
    }
  }
  lds_barrier();
  // diagonal block w: lane j < 16 carries column j of the block
  if (lane < 16) {
    const int q0 = 16 * w, j = lane;
    float tc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float sacc = 0.0f;
#pragma unroll
      for (int m = 0; m < i; ++m) sacc = fmaf(sN[q0 + i][q0 + m], tc[m], sacc);
      tc[i] = i == j ? 1.0f : (j < i ? -sacc : 0.0f);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sT[q0 + i][q0 + j] = tc[i];
  }
  lds_barrier();
  // The blocks below the diagonal, block row by block row, on
  // v_mfma_f32_16x16x4_f32 (fp32 operands and sums, like the substitution):
  // wave J of block row I forms X = sum_{J <= M < I} N_IM T_MJ, passes it
  // through LDS (its rows become the k-runs of the next B operand) and writes
  // T_IJ = -T_II X over N_IJ, once every wave of the row has read its N
  // blocks.  Operand lanes: A[l16][g4], B[g4][l16]; result rows
  // 4 g4 .. 4 g4 + 3 of column l16.  X_J lives in block (J, 3), above the
  // diagonal, which neither N nor T fills (T's upper triangle is read as
  // zero).
  for (int I = 1; I < C / 16; ++I) {
    if (w < I) {
      const int J = w;
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int M = J; M < I; ++M) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          x = __builtin_amdgcn_mfma_f32_16x16x4f32(sN[16 * I + l16][16 * M + 4 * kk + g4],
                                                    sT[16 * M + 4 * kk + g4][16 * J + l16], x, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sT[16 * J + 4 * g4 + r][48 + l16] = x[r];
    }
    lds_barrier();  // every N_IM of the row read
    if (w < I) {
      const int J = w;
      f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        y = __builtin_amdgcn_mfma_f32_16x16x4f32(sT[16 * I + l16][16 * I + 4 * kk + g4],
                                                  sT[16 * J + 4 * kk + g4][48 + l16], y, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) sT[16 * I + 4 * g4 + r][16 * J + l16] = -y[r];
    }
    lds_barrier();
  }
  // The lane's row io = 16w + l16 of the left factor T diag(f) as bf16 high
  // and remainder parts, over token steps s (the B operands of the W and U0
  // products; T is lower triangular): columns 32s + 8 g4 .. + 7.
  const int io = 16 * w + l16;  // the row this lane forms and stores
  auto split_row = [&](bool with_decay, u32x4 (&th)[C / 32], u32x4 (&tl)[C / 32]) {
#pragma unroll
    for (int s = 0; s < C / 32; ++s) {
      uint32_t hp[4], lp[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int m = 32 * s + 8 * g4 + e;
        float f0 = sbeta[m], f1 = sbeta[m + 1];
        if (with_decay) {
          f0 *= ex2(sb[m]);
          f1 *= ex2(sb[m + 1]);
        }
        const float x0 = m <= io ? sT[io][m] * f0 : 0.0f;
        const float x1 = m + 1 <= io ? sT[io][m + 1] * f1 : 0.0f;
        const uint32_t hi = cvt2(x0, x1);
        hp[e / 2] = hi;
        lp[e / 2] = cvt2(x0 - bf16_to_f32(hi & 0xffffu), x1 - bf16_to_f32(hi >> 16));
      }
      th[s] = u32x4{hp[0], hp[1], hp[2], hp[3]};
      tl[s] = u32x4{lp[0], lp[1], lp[2], lp[3]};
    }
  };
  u32x4 th[C / 32], tl[C / 32];
  split_row(true, th, tl);
  // W = (T diag(beta e^b)) K: wave w, rows 16w .., every 16-column tile of the
  // keys.  Formed transposed (K^T as the A operand): lane (l16, g4) then holds
  // columns 4 g4 .. 4 g4 + 3 of row 16w + l16, one 8-byte store.
  uint16_t* wo = reinterpret_cast<uint16_t*>(a.ws_W) + rowk * DK;
  for (int nt = 0; nt < DK / 16; ++nt) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C / 32; ++s) {
      const u32x4 ak = lds_tr8(sK, QS, 32 * s + 8 * g4, 16 * nt, l16);
      acc = mfma16x16x32(ak, th[s], acc);
      acc = mfma16x16x32(ak, tl[s], acc);
    }
    if (io < n)
      *reinterpret_cast<uint2*>(wo + (size_t)io * DK + 16 * nt + 4 * g4) =
          make_uint2(cvt2(acc[0], acc[1]), cvt2(acc[2], acc[3]));
  }
  lds_barrier();  // W has read the K tile: V takes its place
#pragma unroll
  for (int p = 0; p < PV; ++p) {
    const int idx = min(tid + 256 * p, C * VCH - 1), row = idx / VCH, ch = idx % VCH;
    *reinterpret_cast<u32x4*>(&sV[row * VS + 8 * ch]) = (whole_chunk || row < n) ? xv[p] : zero4;
  }
  split_row(false, th, tl);
  lds_barrier();  // the V tile stored
  // U0 = (T diag(beta)) V, bf16 like W and formed transposed the same way
  uint16_t* uo = reinterpret_cast<uint16_t*>(a.ws_U) + rowk * DV;
  for (int nt = 0; nt < DV / 16; ++nt) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C / 32; ++s) {
      const u32x4 av = lds_tr8(sV, VS, 32 * s + 8 * g4, 16 * nt, l16);
      acc = mfma16x16x32(av, th[s], acc);
      acc = mfma16x16x32(av, tl[s], acc);
    }
    if (io < n)
      *reinterpret_cast<uint2*>(uo + (size_t)io * DV + 16 * nt + 4 * g4) =
          make_uint2(cvt2(acc[0], acc[1]), cvt2(acc[2], acc[3]));
  }
}

// 16-byte-chunk XOR swizzle of a row-major bf16 tile with WC chunks per row
// (no padding, so that one 64-lane tile copy fills 1 KB of consecutive LDS):
// chunk p of row r holds the row's chunk p ^ ((r / R) mod WC), R the rows per
// 256-byte bank line, so 16 consecutive rows read at one logical column land
// in 16 distinct bank groups.  Byte offset of element (row, col).
template <int WC>
__device__ __forceinline__ int dswz(int row, int col) {
  constexpr int R = WC >= 16 ? 1 : 16 / WC;
  const int chunk = (col >> 3) ^ ((row / R) & (WC - 1));
  return row * (WC * 16) + (chunk << 4) + ((col & 7) << 1);
}
// The 16-byte chunk of a tile copy's lane: slot q (row q / WC, LDS chunk
// q mod WC) holds the row's chunk p ^ ((row / R) mod WC).
template <int WC>
__device__ __forceinline__ int dswz_src_chunk(int q) {
  constexpr int R = WC >= 16 ? 1 : 16 / WC;
  const int r = q / WC, p = q % WC;
  return p ^ ((r / R) & (WC - 1));
}
// lds_tr8 on a swizzled tile of WC chunks per row
template <int WC>
__device__ __forceinline__ u32x4 lds_tr8s(const char* base, int k0, int col0, int l16) {
  const int j = l16 >> 2, m = l16 & 3;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(base + dswz<WC>(k0 + j, col0 + 4 * m)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(base + dswz<WC>(k0 + 4 + j, col0 + 4 * m)));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return u32x4{a[0], a[1], b[0], b[1]};
}
__device__ __forceinline__ u32x4 lds_b128(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
// s_waitcnt with only the vector-memory count set: at most N vector memory
// instructions of this wave may be outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The sequential pass for bf16 inputs on v_mfma_f32_16x16x32_bf16: one
// workgroup of 4 waves per (head, TV value columns), C = 64.  Wave w owns
// the chunk's query rows 16w .. 16w + 15 and the state rows (keys) of 16-row
// tiles w, w + 4, ...; the state tile lives in its fp32
// accumulators, with a bf16 copy S^T in LDS (double-buffered by chunk parity)
// as the B operand of W S and Q S.  Per chunk:
//   (1) U = U0 - W S for the wave's rows -> U^T and (e^{b_last - b} U)^T in
//       LDS (bf16); the chunk's masked, decayed scores P come ready from the
//       solve pass (bf16 rows in the workspace), so no score products sit on
//       this pass's chunk-to-chunk critical path;
//   (2) O = diag(e^b) Q S + P U for the wave's rows -> HBM; the state update
//       S = e^{b_last} S + K^T (e^{b_last - b} U), the K^T operand read from
//       the row-major K tile with transpose reads; the new S^T to the other
//       LDS buffer.
// The chunk's q, k, W, P and U0 tiles and its decay prefix b (from the solve
// pass) go from memory straight into LDS with global_load_lds (two stages:
// the next chunk's copies fly while the current one computes).  The loop
// then holds no register loads, whose completion the compiler would wait for
// by draining every outstanding memory operation, the previous chunk's
// output stores included; its one wait for memory counts instructions.  Rows
// past a short last chunk are copies of its last row: they meet zero weights
// in the state update and give outputs that are not stored.
template <int DK, int TV>
__global__ __launch_bounds__(256) void delta_chunk_mfma_kernel(const DeltaArgs a) {
  constexpr int C = 64;
  constexpr int NT = TV / 16;       // 16-column tiles of the value columns
  constexpr int QS = DK + 8;        // bf16 row stride of S^T
  constexpr int CS = C + 8;         // bf16 row stride of U^T
  constexpr int KST = DK / 32;      // 32-wide k-steps over the keys
  constexpr int NMT = DK / 16;      // 16-row tiles of the state
  constexpr int MTW = (NMT + 3) / 4;
  constexpr int NWV = 4;            // waves of the workgroup
  constexpr int WCQ = DK / 8;       // 16-byte chunks of a q / k / W row
  constexpr int WCP = C / 8;        // ... of a score row
  constexpr int WCU = TV / 8;       // ... of a U0 row
  constexpr int QB = C * DK * 2, PB = C * C * 2, UB = C * TV * 2;  // tile bytes
  // 1 KB tile copies (64 lanes x 16 bytes) per wave and chunk: equal for every
  // wave, so the wait below can count them
  constexpr int QPER = C * WCQ / 64 / NWV;
  constexpr int PPER = C * WCP / 64 / NWV;
  // (the U0 tile is 2 or 4 KB: the first UBLK waves copy one block each;
  // the wait counts only what a wave issues after its copies)
  constexpr int UBLK = C * WCU / 64;
  constexpr int BPER = C / NWV;     // decay prefixes each wave copies
  static_assert(QPER >= 1 && C * WCQ % (64 * NWV) == 0, "q/k/W copies per wave");
  static_assert(PPER >= 1 && C * WCP % (64 * NWV) == 0, "score copies per wave");
  static_assert(UBLK >= 1 && UBLK <= 4 && C * WCU % 64 == 0, "U0 tile copies");
  // vector memory instructions of one chunk per wave: copies, then stores
  constexpr int STORES = NT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wg = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave of the workgroup
  const int w = wg;
  const int l16 = lane & 15, g4 = lane >> 4;
  // workgroup -> (head, value tile): the tiles of one head get workgroup ids
  // that are equal mod 8, so they run on one XCD and share q, k and W
  // through its L2
  const int f = blockIdx.x;
  const int slot = f >> 3;
  const int vt = slot % a.n_v;
  const int bh = (slot / a.n_v) * 8 + (f & 7);
  if (bh >= a.B * a.H) return;
  const int L = a.L, DV = a.DV;
  const int dv0 = vt * TV;
  const int nch = (L + C - 1) / C;

  __shared__ __align__(16) char sQ[2][QB], sK[2][QB], sW[2][QB], sP[2][PB], sU0t[2][UB];
  __shared__ __align__(16) float sb[2][C];
  __shared__ __align__(16) uint16_t sST[2][TV * QS];
  __shared__ __align__(16) uint16_t sUT[TV * CS], sUwT[TV * CS];

  const uint16_t* qh = static_cast<const uint16_t*>(a.q) + (size_t)bh * L * DK;
  const uint16_t* kh = static_cast<const uint16_t*>(a.k) + (size_t)bh * L * DK;
  const uint16_t* wh = reinterpret_cast<const uint16_t*>(a.ws_W) + (size_t)bh * L * DK;
  const uint16_t* ph = static_cast<const uint16_t*>(a.ws_P) + (size_t)bh * L * C;
  const uint16_t* uh = reinterpret_cast<const uint16_t*>(a.ws_U) + (size_t)bh * L * DV + dv0;
  const float* bhp = a.ws_b + (size_t)bh * L;
  uint16_t* oh = static_cast<uint16_t*>(a.out) + (size_t)bh * L * DV + dv0;

  // per-lane sources of the tile copies, relative to the chunk's first row
  int qrow[QPER], qoff[QPER], prow[PPER], poff[PPER];
#pragma unroll
  for (int i = 0; i < QPER; ++i) {
    const int q = 64 * (wg + NWV * i) + lane;
    qrow[i] = q / WCQ;
    qoff[i] = qrow[i] * DK + 8 * dswz_src_chunk<WCQ>(q);
  }
#pragma unroll
  for (int i = 0; i < PPER; ++i) {
    const int q = 64 * (wg + NWV * i) + lane;
    prow[i] = q / WCP;
    poff[i] = prow[i] * C + 8 * dswz_src_chunk<WCP>(q);
  }
  const int urow = (64 * w + lane) / WCU;
  const int uoff = urow * DV + 8 * ((64 * w + lane) % WCU);
  // Copies of chunk c into stage st (rows past the sequence re-read its last
  // row), an equal share per wave.
  auto issue = [&](int c, int st) {
    const int t0 = c * C, last = min(C, L - t0) - 1;
    const bool whole = last == C - 1;
    const size_t rq = (size_t)t0 * DK;
#pragma unroll
    for (int i = 0; i < QPER; ++i) {
      const int off = whole ? qoff[i] : qoff[i] - max(qrow[i] - last, 0) * DK;
      const int dst = 1024 * (wg + NWV * i);
      dma16(qh + rq + off, sQ[st] + dst);
      dma16(kh + rq + off, sK[st] + dst);
      dma16(wh + rq + off, sW[st] + dst);
    }
#pragma unroll
    for (int i = 0; i < PPER; ++i) {
      const int off = whole ? poff[i] : poff[i] - max(prow[i] - last, 0) * C;
      dma16(ph + (size_t)t0 * C + off, sP[st] + 1024 * (wg + NWV * i));
    }
    if (w < UBLK) {
      const int off = whole ? uoff : uoff - max(urow - last, 0) * DV;
      dma16(uh + (size_t)t0 * DV + off, sU0t[st] + 1024 * w);
    }
    if (lane < BPER) dma4(bhp + t0 + min(wg * BPER + lane, last), &sb[st][wg * BPER]);
  };
  // ---- the state: own tiles (mt = w + 4 m, nt), lane rows 16 mt + 4 g4 + r, column 16 nt + l16
  f32x4 accS[MTW][NT];
  auto put_state = [&](int buf) {
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      const int mt = w + 4 * m;
      if (mt < NMT) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          *reinterpret_cast<uint2*>(&sST[buf][(16 * nt + l16) * QS + 16 * mt + 4 * g4]) =
              make_uint2(cvt2(accS[m][nt][0], accS[m][nt][1]), cvt2(accS[m][nt][2], accS[m][nt][3]));
      }
    }
  };
#pragma unroll
  for (int m = 0; m < MTW; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mt = w + 4 * m, d = 16 * mt + 4 * g4 + r;
        accS[m][nt][r] = (a.state && mt < NMT)
                             ? a.state[((size_t)bh * DK + d) * DV + dv0 + 16 * nt + l16]
                             : 0.0f;
      }
  put_state(0);
  if (nch > 0) issue(0, 0);

  for (int c = 0; c < nch; ++c) {
    const int t0 = c * C, n = min(C, L - t0);
    const int sp = c & 1;  // tile stage and S^T buffer of this chunk
    // this wave's copies of chunk c have landed: in issue order they are
    // followed only by the previous chunk's output stores (a whole chunk)
    if (c == 0) wait_vm<0>();
    else wait_vm<STORES>();
    lds_barrier();  // every wave's copies landed; the previous chunk is done; S^T[sp] complete
    if (c + 1 < nch) issue(c + 1, sp ^ 1);
    const char* cQ = sQ[sp];
    const char* cK = sK[sp];
    const char* cW = sW[sp];
    const char* cP = sP[sp];
    const uint16_t* sU0 = reinterpret_cast<const uint16_t*>(sU0t[sp]);
    const float* cb = sb[sp];
    const float bL = cb[n - 1];
    const uint16_t* st = sST[sp];

    // (1a) U = U0 - W S for rows 16w .. 16w + 15, and with it (sharing the S
    // operand reads, ahead of the barrier the rest of O waits behind) the
    // part of O that does not wait for U, Q S for the same rows.  O is formed
    // transposed (S^T, U^T rows as the A operand): lane (l16, g4) then holds
    // value columns 4 g4 .. 4 g4 + 3 of token 16w + l16, one 8-byte store.
    f32x4 accO[NT];
    {
      f32x4 acc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        accO[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int s = 0; s < KST; ++s) {
        const u32x4 aw = lds_b128(cW, dswz<WCQ>(16 * w + l16, 32 * s + 8 * g4));
        const u32x4 aq = lds_b128(cQ, dswz<WCQ>(16 * w + l16, 32 * s + 8 * g4));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const u32x4 bs = *reinterpret_cast<const u32x4*>(&st[(16 * nt + l16) * QS + 32 * s + 8 * g4]);
          acc[nt] = mfma16x16x32(aw, bs, acc[nt]);
          accO[nt] = mfma16x16x32(bs, aq, accO[nt]);
        }
      }
      const int i0 = 16 * w + 4 * g4;
      float wt[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) wt[r] = i0 + r < n ? ex2(bL - cb[i0 + r]) : 0.0f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float u[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) u[r] = bf16_to_f32(sU0[(i0 + r) * TV + 16 * nt + l16]) - acc[nt][r];
        const int o = (16 * nt + l16) * CS + i0;
        *reinterpret_cast<uint2*>(&sUT[o]) = make_uint2(cvt2(u[0], u[1]), cvt2(u[2], u[3]));
        *reinterpret_cast<uint2*>(&sUwT[o]) = make_uint2(cvt2(u[0] * wt[0], u[1] * wt[1]),
                                                         cvt2(u[2] * wt[2], u[3] * wt[3]));
      }
    }
    lds_barrier();  // U^T and (wU)^T complete

    // (2a) O = diag(e^b) Q S + P U for rows 16w .. 16w + 15
    {
      const int io = 16 * w + l16;  // this lane's token
      const float e = ex2(cb[io]);
      f32x4 acc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = accO[nt] * e;
      // token k-steps up to the diagonal: rows 16w .. need tokens < 16w + 16
      for (int s2 = 0; s2 <= w / 2; ++s2) {
        const u32x4 ap = lds_b128(cP, dswz<WCP>(io, 32 * s2 + 8 * g4));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const u32x4 bu = *reinterpret_cast<const u32x4*>(&sUT[(16 * nt + l16) * CS + 32 * s2 + 8 * g4]);
          acc[nt] = mfma16x16x32(bu, ap, acc[nt]);
        }
      }
      if (io < n) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          *reinterpret_cast<uint2*>(oh + (size_t)(t0 + io) * DV + 16 * nt + 4 * g4) =
              make_uint2(cvt2(acc[nt][0], acc[nt][1]), cvt2(acc[nt][2], acc[nt][3]));
      }
    }
    // (2b) S = e^{b_last} S + K^T (e^{b_last - b} U) for the wave's state tiles
    {
      const float eL = ex2(bL);
#pragma unroll
      for (int m = 0; m < MTW; ++m) {
        const int mt = w + 4 * m;
        if (mt < NMT) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            f32x4 acc = accS[m][nt] * eL;
#pragma unroll
            for (int s2 = 0; s2 < C / 32; ++s2) {
              const u32x4 ak = lds_tr8s<WCQ>(cK, 32 * s2 + 8 * g4, 16 * mt, l16);
              const u32x4 bu = *reinterpret_cast<const u32x4*>(&sUwT[(16 * nt + l16) * CS + 32 * s2 + 8 * g4]);
              acc = mfma16x16x32(ak, bu, acc);
            }
            accS[m][nt] = acc;
          }
        }
      }
      put_state(sp ^ 1);
    }
  }
  if (a.state) {
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      const int mt = w + 4 * m;
      if (mt < NMT) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            a.state[((size_t)bh * DK + 16 * mt + 4 * g4 + r) * DV + dv0 + 16 * nt + l16] = accS[m][nt][r];
      }
    }
  }
}

// The column pass below keeps its state and U as fp32 accumulator tiles and
// feeds them to the next products as operands after rounding to bf16 alone,
// with no exchange between lanes.  A 16x16x32 product sums over its 32 k
// indices in any order both operands agree on, so the keys (of S) and the
// tokens (of U) are numbered in the order in which two 16x16 accumulator
// tiles hold their rows: within each 32-wide k-step (s or t), tile 2s + h row
// 4a + b is index 8a + 4h + b (a, b < 4).  Lane (l16, g4) of a tile pair then
// holds indices 8 g4 .. 8 g4 + 7 of the k-step, in order, as an operand wants
// them; the row tiles read from LDS take the same numbering (row l16 of
// tile 2t + h is token 32t + 8 (l16 / 4) + 4h + l16 % 4).
__device__ __forceinline__ u32x4 pack_pair(const f32x4& t0, const f32x4& t1) {
  return u32x4{cvt2(t0[0], t0[1]), cvt2(t0[2], t0[3]), cvt2(t1[0], t1[1]), cvt2(t1[2], t1[3])};
}
__device__ __forceinline__ int perm_index(int k0, int h, int l16) {
  return k0 + 8 * (l16 >> 2) + 4 * h + (l16 & 3);
}
// 16-byte-chunk XOR swizzles of bf16 tiles with WC (8 or 16) chunks per row,
// one per access pattern of that pass (physical chunk = logical chunk ^
// swizzle(row)), each making the 16 lanes of a quarter-wave hit distinct
// banks.  Rows: lanes read rows perm_index(.., l16) at one column (the q, W
// and score tiles).  Cols: lanes (j, m) = (l16 / 4, l16 % 4) read row k0 + j
// (k0 a multiple of 4) at chunk 4s + m (transpose reads of the k tile).
template <int WC>
__device__ __forceinline__ int swz_rows(int row) {
  static_assert(WC == 8 || WC == 16, "8 or 16 chunks per row");
  if constexpr (WC == 16) return (row & 3) | ((row >> 1) & 12);
  else return ((row >> 1) & 1) | ((row >> 2) & 6);
}
template <int WC>
__device__ __forceinline__ int swz_cols(int row) {
  static_assert(WC == 8 || WC == 16, "8 or 16 chunks per row");
  if constexpr (WC == 16) return (row & 3) << 2;
  else return ((row >> 1) & 1) << 2;
}
// byte offset of element (row, col); the logical chunk a tile copy's slot q
// (row q / WC, physical chunk q % WC) holds
template <int WC, bool ROWS>
__device__ __forceinline__ int off_sw(int row, int col) {
  const int sw = ROWS ? swz_rows<WC>(row) : swz_cols<WC>(row);
  return row * (WC * 16) + (((col >> 3) ^ sw) << 4) + ((col & 7) << 1);
}
template <int WC, bool ROWS>
__device__ __forceinline__ int src_sw(int q) {
  const int row = q / WC;
  return (q % WC) ^ (ROWS ? swz_rows<WC>(row) : swz_cols<WC>(row));
}
// K^T as the A operand of key tile 2s + h over token step k0 + 8 g4 .. + 7:
// lane (l16, g4) gets key perm_index(32 s, h, l16) at those 8 tokens
template <int WC>
__device__ __forceinline__ u32x4 lds_ktr(const char* base, int k0, int s, int h, int l16) {
  const int j = l16 >> 2, m = l16 & 3, c = 32 * s + 8 * m + 4 * h;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off_sw<WC, false>(k0 + j, c)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off_sw<WC, false>(k0 + 4 + j, c)));
  const u32x2 x = __builtin_bit_cast(u32x2, lo), y = __builtin_bit_cast(u32x2, hi);
  return u32x4{x[0], x[1], y[0], y[1]};
}

// The sequential pass by value columns, for workgroups of 32 value columns
// (d_k >= 64).  The recurrence never mixes value columns: U = U0 - W S, O and
// the update of S for columns j need only S's columns j.  Each of waves 0-1
// so carries the whole chunk-to-chunk chain for its 16 columns in its own
// registers, with no barrier between U and the state update: its state
// tiles are fp32 accumulators (keys numbered as above), and the products
// take the accumulators of S and U as operands.  Waves 2-5 move the tiles:
// at the top of chunk c they store chunk c + 1's tiles (loaded into
// registers a chunk earlier) to the other LDS stage and issue chunk c + 2's
// loads.  One barrier per chunk (tiles stored, the previous chunk's tiles
// free).
template <int DK>
__global__ __launch_bounds__(384) void delta_chunk_cols_kernel(const DeltaArgs a) {
  constexpr int C = 64, TV = 32;
  constexpr int KST = DK / 32;      // 32-wide k-steps over the keys
  constexpr int NMT = DK / 16;      // 16-row key tiles of the state
  constexpr int WCQ = DK / 8;       // 16-byte chunks of a q / k / W row
  constexpr int WCP = C / 8;        // ... of a score row
  constexpr int WCU = TV / 8;       // ... of a U0 row
  constexpr int QB = C * DK * 2, PB = C * C * 2, UB = C * TV * 2;  // tile bytes
  // 1 KB blocks per copying wave and chunk, of each q / k / W tile, of the
  // score tile and of the U0 tile
  constexpr int QPER = C * WCQ / 64 / 4;
  constexpr int PPER = C * WCP / 64 / 4;
  constexpr int UPER = C * WCU / 64 / 4;
  static_assert(DK == 64 || DK == 128, "d_k of the column pass");
  static_assert(QPER >= 1 && PPER >= 1 && UPER >= 1, "tile copies per copying wave");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wg = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool copier = wg >= 2;
  const int w = copier ? wg - 2 : wg;  // copying wave, or the compute wave's 16-column half
  const int l16 = lane & 15, g4 = lane >> 4;
  // workgroup -> (head, value tile) as in the pass above
  const int f = blockIdx.x;
  const int slot = f >> 3;
  const int vt = slot % a.n_v;
  const int bh = (slot / a.n_v) * 8 + (f & 7);
  if (bh >= a.B * a.H) return;
  const int L = a.L, DV = a.DV;
  const int dv0 = vt * TV;
  const int nch = (L + C - 1) / C;

  __shared__ __align__(16) char sQ[2][QB], sK[2][QB], sW[2][QB], sP[2][PB], sU0[2][UB];
  __shared__ __align__(16) float sb[2][C];

  const uint16_t* qh = static_cast<const uint16_t*>(a.q) + (size_t)bh * L * DK;
  const uint16_t* kh = static_cast<const uint16_t*>(a.k) + (size_t)bh * L * DK;
  const uint16_t* wh = reinterpret_cast<const uint16_t*>(a.ws_W) + (size_t)bh * L * DK;
  const uint16_t* ph = static_cast<const uint16_t*>(a.ws_P) + (size_t)bh * L * C;
  const uint16_t* uh = reinterpret_cast<const uint16_t*>(a.ws_U) + (size_t)bh * L * DV + dv0;
  const float* bhp = a.ws_b + (size_t)bh * L;

  if (copier) {
    // copying wave w's share of chunk c's tiles: 1 KB blocks w, w + 4, ..
    // of each, loaded into registers (rows past the sequence re-read its
    // last row) and stored to a tile stage a chunk later, each lane's 16
    // bytes at 16 lane.  These waves issue no stores to memory, so the waits
    // for these loads cover nothing else.
    u32x4 xw[QPER], xq[QPER], xk[QPER], xu[UPER], xp[PPER];
    float xb = 0.0f;
    auto fetch = [&](int c) {
      const int t0 = c * C, last = min(C, L - t0) - 1;
      const size_t rq = (size_t)t0 * DK;
#pragma unroll
      for (int i = 0; i < QPER; ++i) {
        const int q = 64 * (w + 4 * i) + lane;
        const int row = min(q / WCQ, last) * DK;
        xw[i] = *reinterpret_cast<const u32x4*>(wh + rq + row + 8 * src_sw<WCQ, true>(q));
        xq[i] = *reinterpret_cast<const u32x4*>(qh + rq + row + 8 * src_sw<WCQ, true>(q));
        xk[i] = *reinterpret_cast<const u32x4*>(kh + rq + row + 8 * src_sw<WCQ, false>(q));
      }
#pragma unroll
      for (int i = 0; i < UPER; ++i) {
        const int q = 64 * (w + 4 * i) + lane;
        const int off = min(q / WCU, last) * DV + 8 * (q % WCU);
        xu[i] = *reinterpret_cast<const u32x4*>(uh + (size_t)t0 * DV + off);
      }
#pragma unroll
      for (int i = 0; i < PPER; ++i) {
        const int q = 64 * (w + 4 * i) + lane;
        const int off = min(q / WCP, last) * C + 8 * src_sw<WCP, true>(q);
        xp[i] = *reinterpret_cast<const u32x4*>(ph + (size_t)t0 * C + off);
      }
      xb = bhp[t0 + min(lane, last)];
    };
    auto stash = [&](int st) {
#pragma unroll
      for (int i = 0; i < QPER; ++i) {
        const int o = 1024 * (w + 4 * i) + 16 * lane;
        *reinterpret_cast<u32x4*>(sW[st] + o) = xw[i];
        *reinterpret_cast<u32x4*>(sQ[st] + o) = xq[i];
        *reinterpret_cast<u32x4*>(sK[st] + o) = xk[i];
      }
#pragma unroll
      for (int i = 0; i < UPER; ++i)
        *reinterpret_cast<u32x4*>(sU0[st] + 1024 * (w + 4 * i) + 16 * lane) = xu[i];
#pragma unroll
      for (int i = 0; i < PPER; ++i)
        *reinterpret_cast<u32x4*>(sP[st] + 1024 * (w + 4 * i) + 16 * lane) = xp[i];
      if (w == 0) sb[st][lane] = xb;
    };
    if (nch > 0) {
      fetch(0);
      stash(0);
    }
    if (nch > 1) fetch(1);
    for (int c = 0; c < nch; ++c) {
      lds_barrier();  // chunk c's tiles stored; chunk c - 1's stage is free
      if (c + 1 < nch) stash((c & 1) ^ 1);
      if (c + 2 < nch) fetch(c + 2);
    }
    return;
  }

  // ---- compute wave w: value column dv0 + 16 w + l16 (the lane's column)
  const int col = 16 * w + l16;  // within the workgroup's 32
  // state tile 2s + h: lane rows are keys 32 s + 8 g4 + 4 h + r
  f32x4 accS[NMT];
#pragma unroll
  for (int m = 0; m < NMT; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 32 * (m >> 1) + 8 * g4 + 4 * (m & 1) + r;
      accS[m][r] = a.state ? a.state[((size_t)bh * DK + key) * DV + dv0 + col] : 0.0f;
    }
  uint16_t* oh = static_cast<uint16_t*>(a.out) + (size_t)bh * L * DV + dv0 + 16 * w;

  for (int c = 0; c < nch; ++c) {
    const int t0 = c * C, n = min(C, L - t0);
    const int sp = c & 1;
    lds_barrier();  // chunk c's tiles stored
    const char* cQ = sQ[sp];
    const char* cK = sK[sp];
    const char* cW = sW[sp];
    const char* cP = sP[sp];
    const uint16_t* cU0 = reinterpret_cast<const uint16_t*>(sU0[sp]);
    const float* cb = sb[sp];
    const float bL = cb[n - 1];

    // The LDS reads are issued in batches ahead of the products that use
    // them (scheduling barriers keep each batch ahead of the products of the
    // batch before): with one wave per SIMD nothing else hides their
    // latency, and left alone the compiler waits for each read right before
    // its product.
    // (a) what U, the state's weights and O's scaling need
    uint32_t u0v[4][4];
    f32x4 bt[4];
    float bo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tk = 32 * (i >> 1) + 8 * g4 + 4 * (i & 1);  // + r: token of U row r
#pragma unroll
      for (int r = 0; r < 4; ++r) u0v[i][r] = cU0[(tk + r) * TV + col];
      bt[i] = *reinterpret_cast<const f32x4*>(&cb[tk]);
      bo[i] = cb[perm_index(32 * (i >> 1), i & 1, l16)];
    }
    // (1) W S for token tiles i (lane rows: tokens perm_index(32 (i / 2),
    // i % 2, 4 g4 + r), the lane's column) and, sharing the S operand,
    // (Q S)^T (value columns 4 g4 + r of the wave's 16, token
    // perm_index(.., l16)), key step s's operands read a step ahead
    u32x4 aw[2][4], aq[2][4];
    auto read_wq = [&](int s, int buf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = off_sw<WCQ, true>(perm_index(32 * (i >> 1), i & 1, l16), 32 * s + 8 * g4);
        aw[buf][i] = *reinterpret_cast<const u32x4*>(cW + o);
        aq[buf][i] = *reinterpret_cast<const u32x4*>(cQ + o);
      }
    };
    read_wq(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    // S as operand over key step s
    u32x4 bS[KST];
#pragma unroll
    for (int s = 0; s < KST; ++s) bS[s] = pack_pair(accS[2 * s], accS[2 * s + 1]);
    f32x4 accU[4], accO[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      accU[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      accO[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // the K^T operands of (2), key tiles m0 .. m0 + NMT/2 - 1
    constexpr int MH = NMT / 2;
    u32x4 ak[MH][2], ap[6];
    auto read_k = [&](int m0) {
#pragma unroll
      for (int m = 0; m < MH; ++m)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          ak[m][t] = lds_ktr<WCQ>(cK, 32 * t + 8 * g4, (m0 + m) >> 1, (m0 + m) & 1, l16);
    };
#pragma unroll
    for (int s = 0; s < KST; ++s) {
      if (s + 1 < KST) read_wq(s + 1, (s + 1) & 1);
      else read_k(0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        accU[i] = mfma16x16x32(aw[s & 1][i], bS[s], accU[i]);
        accO[i] = mfma16x16x32(bS[s], aq[s & 1][i], accO[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // U = U0 - W S and the state's weights e^{b_last - b} U (zero past the
    // sequence), as operands over token step t (tiles 2t, 2t + 1)
    u32x4 bU[2], bwU[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 u[2], uw[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = 2 * t + h, tk = 32 * t + 8 * g4 + 4 * h;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          u[h][r] = bf16_to_f32(u0v[i][r]) - accU[i][r];
          uw[h][r] = tk + r < n ? u[h][r] * ex2(bL - bt[i][r]) : 0.0f;
        }
      }
      bU[t] = pack_pair(u[0], u[1]);
      bwU[t] = pack_pair(uw[0], uw[1]);
    }

    // (2) S = e^{b_last} S + K^T (e^{b_last - b} U), in two halves of the
    // key tiles; the second half's operands and the score operands of (3)
    // are read while the first half's products run
    const float eL = ex2(bL);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if (hf == 1) {
        read_k(MH);
#pragma unroll
        for (int i = 0, x = 0; i < 4; ++i)
#pragma unroll
          for (int t = 0; t <= i / 2; ++t, ++x)
            ap[x] = *reinterpret_cast<const u32x4*>(
                cP + off_sw<WCP, true>(perm_index(32 * (i >> 1), i & 1, l16), 32 * t + 8 * g4));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < MH; ++m) {
        f32x4 acc = accS[MH * hf + m] * eL;
#pragma unroll
        for (int t = 0; t < 2; ++t) acc = mfma16x16x32(ak[m][t], bwU[t], acc);
        accS[MH * hf + m] = acc;
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // (3) O^T = diag(e^b) (Q S)^T + U^T P^T: token perm_index(.., l16), value
    // columns 4 g4 .. 4 g4 + 3 of the wave's 16 (one 8-byte store)
#pragma unroll
    for (int i = 0, x = 0; i < 4; ++i) {
      const int io = perm_index(32 * (i >> 1), i & 1, l16);
      f32x4 acc = accO[i] * ex2(bo[i]);
#pragma unroll
      for (int t = 0; t <= i / 2; ++t, ++x) acc = mfma16x16x32(bU[t], ap[x], acc);
      if (io < n)
        *reinterpret_cast<uint2*>(oh + (size_t)(t0 + io) * DV + 4 * g4) =
            make_uint2(cvt2(acc[0], acc[1]), cvt2(acc[2], acc[3]));
    }
  }
  if (a.state) {
#pragma unroll
    for (int m = 0; m < NMT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 32 * (m >> 1) + 8 * g4 + 4 * (m & 1) + r;
        a.state[((size_t)bh * DK + key) * DV + dv0 + col] = accS[m][r];
      }
  }
}

// The sequential MFMA pass: 32 value columns per workgroup; where 4-wave
// 32-column workgroups would leave fewer than two per compute unit of an
// MI355X (256 of them), the column pass instead (d_k >= 64: two waves that
// each carry 16 columns' whole chain, four that move the tiles).
template <int D>
void launch_chunk_mfma(const DeltaArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (D >= 64) {
    if ((long long)a.B * a.H * a.n_v < 512) {
      hipLaunchKernelGGL((delta_chunk_cols_kernel<D>), grid, dim3(384), 0, s, a);
      return;
    }
  }
  if (a.n_v == a.DV / 16)
    hipLaunchKernelGGL((delta_chunk_mfma_kernel<D, 16>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((delta_chunk_mfma_kernel<D, 32>), grid, dim3(256), 0, s, a);
}

template <bool BF16>
hipError_t launch_dk(const DeltaArgs& a, hipStream_t s) {
  const int nch = (a.L + a.C - 1) / a.C;
  const dim3 gp(a.B * a.H * nch), gc(a.B * a.H * a.n_v), blk(256);
  // the MFMA pass numbers its workgroups by groups of 8 heads (see there)
  const dim3 gm(((a.B * a.H + 7) / 8) * 8 * a.n_v);
  // bf16 inputs, C = 64, d_k >= 32 and whole 32-column value tiles: the MFMA pass
  const bool mfma = BF16 && delta_uses_mfma(a.dtype, a.C, a.DK, a.DV);
  switch (a.DK) {
#define LA_DK(D)                                                                  \
  case D:                                                                         \
    if constexpr (BF16 && D >= 32) {                                              \
      if (mfma) {                                                                 \
        hipLaunchKernelGGL((delta_prep_mfma_kernel<D>), gp, blk, 0, s, a);        \
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;        \
        launch_chunk_mfma<D>(a, gm, s);                                           \
        return hipGetLastError();                                                 \
      }                                                                           \
    }                                                                             \
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
  int tv = a.DV < kDeltaTile ? a.DV : kDeltaTile;
  // the MFMA pass: 16-column 4-wave workgroups where d_k < 64 would leave
  // fewer than two 32-column workgroups per compute unit (see launch_chunk_mfma)
  if (delta_uses_mfma(a.dtype, a.C, a.DK, a.DV) && a.DK < 64 &&
      (long long)a.B * a.H * (a.DV / 32) < 512)
    tv = 16;
  b.n_v = a.DV / tv;
  return a.dtype == kBF16 ? launch_dk<true>(b, s) : launch_dk<false>(b, s);
}

}  // namespace la
