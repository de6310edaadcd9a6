// la_chunk_bf16.hip -- chunkwise causal linear attention, bf16 in, gfx950 MFMA.
//
// What one workgroup computes.  A work unit is one head (b, h), one tile of
// TV value columns [dv0, dv0 + TV) and one segment of consecutive chunks of
// the sequence.  For every chunk of C tokens, with b_i the inclusive prefix
// sum of log a over the chunk (every factor below is exp of a value <= 0):
//
//   O_c     = diag(e^b) Q_c S_c + ((Q_c K_c^T) o D_c) V_c,   D_c[i,j] = e^{b_i - b_j} [j <= i]
//   S_{c+1} = e^{b_last} S_c + (diag(e^{b_last - b}) K_c)^T V_c
//
// This is the chunkwise form of "Linear / Sparse Attention - minimal runnable
// implementation" (linear_attn_chunkwise: inter = Q_c S, intra = masked
// (Q_c K_c^T) V_c, then S += K_c^T V_c, ragged last chunk) with the decay
// folded into S_c and the in-chunk mask as the linear/sparse attention
// tutorial's section 6.2 says the gated variants do; the per-element decay
// matrix is the log-space construction of CS336 lecture 4 code 1,
// gated_linear_attention_parallel (log D[t,s] = cumsum[t] - cumsum[s]).
//
// Mapping onto gfx950 (4 waves of 64 lanes, v_mfma_f32_16x16x32_bf16):
//   * the C query rows of a chunk are split into 16-row strips, strip st
//     belongs to wave st % 4.  A wave computes its strip's scores against key
//     blocks 0..st only (the causal upper blocks are skipped), masks and
//     decays them in fp32 registers, and uses them straight from registers as
//     the B operand of the P.V product: the scores come out of the QK^T MFMA
//     transposed (K is the A operand), which is already the operand layout.
//     The 32 token indices of one MFMA k-step are permuted consistently in
//     both operands, so no register shuffle is needed.
//   * the state tile S[:, dv0:dv0+TV] lives in fp32 MFMA accumulators, split
//     over the 4 waves by 16x16 tile; after each update a bf16 copy S^T is
//     written to LDS for the next chunk's inter-chunk product.
//   * K (row-major, for QK^T), K scaled by e^{b_last - b} and transposed (for
//     the state update) and V^T are staged in LDS; Q goes straight from HBM
//     into the B-operand registers of its wave.
//   * the next chunk's K, V, Q and decay values are loaded into registers
//     while the current chunk computes.
//   * the workgroups of one (head, segment) that differ only in the value
//     tile are numbered so that they land on one XCD and share Q and K
//     through that XCD's L2.
//
// A state-only variant (STATE_ONLY) computes, for one segment, the state
// increment dS = sum_t e^{B_end - B_t} k_t v_t^T from a zero state and the
// segment's total log decay; the main pass then starts every segment from
// S_in = e^{A_{s-1}} (... (e^{A_0} S_0 + dS_0) ...) + dS_{s-1}, the prefix of
// the associative (decay, state) composition (the parallel / associative
// scan idea of the tutorial's section 3.3 applied to these pairs).
#include "la_device.h"

namespace la {
namespace {

template <int DK, int TV, int C>
struct Geo {
  static constexpr int CP = C < 32 ? 32 : C;       // chunk padded to whole MFMA k-steps
  static constexpr int DKP = DK < 32 ? 32 : DK;    // key dim padded likewise
  static constexpr int KSTEPS = DKP / 32;          // k-steps over the key dim
  static constexpr int CSTEPS = CP / 32;           // k-steps over the chunk's tokens
  static constexpr int KS = DKP + 8;               // row stride of sK and sST (elements)
  static constexpr int TS = CP + 8;                // row stride of sKT and sVT
  static constexpr int NSTRIP = C / 16;            // 16-row query strips per chunk
  static constexpr int SPW = (NSTRIP + 3) / 4;     // strips per wave
  static constexpr int NTV = TV / 16;              // 16-wide value tiles
  static constexpr int NT_S = (DK / 16) * NTV;     // 16x16 tiles of the state
  static constexpr int TPW = (NT_S + 3) / 4;       // state tiles per wave
  static constexpr int KPIECES = (C / 4) * (DK / 8);  // 4 tokens x 8 dims pieces of K
  static constexpr int VPIECES = (C / 4) * (TV / 8);  // ... of the V tile
  static constexpr int KIT = (KPIECES + 255) / 256;
  static constexpr int VIT = (VPIECES + 255) / 256;
  static constexpr size_t LDS_MAIN =
      2 * ((size_t)C * KS + (size_t)DK * TS + (size_t)TV * TS + 2 * (size_t)TV * KS) + 8 * CP;
};

constexpr size_t kMaxLds = 160 * 1024;

// Storage position of chunk-local token c in the transposed tiles: inside each
// 32-token block, token 16h + 4g + i goes to 8g + 4h + i, so that the 8 values
// an MFMA lane group g holds for one k-step are contiguous.
__device__ __forceinline__ int tok_pos(int c) {
  return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}

__device__ __forceinline__ u32x4 lds16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

template <int DK, int TV, int C, bool STATE_ONLY>
__global__ __launch_bounds__(256) void chunk_bf16_kernel(const ChunkArgs a) {
  using G = Geo<DK, TV, C>;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;

  // workgroup -> (unit, value tile); the tiles of one unit share an XCD
  const int f = blockIdx.x;
  const int slot = f >> 3;
  const int vt = slot % a.n_v;
  const int u = (slot / a.n_v) * 8 + (f & 7);
  if (u >= a.n_units) return;
  const int segs = STATE_ONLY ? a.P - 1 : a.P;
  const int bh = u / segs, sigma = u % segs;
  const int h = bh % a.H;
  const int dv0 = vt * TV;
  const int L = a.L, DV = a.DV;
  const int nchunks = (L + C - 1) / C;
  const int c_begin = sigma * a.seg_chunks;
  const int c_end = min(c_begin + a.seg_chunks, nchunks);
  const int kind = a.decay_kind;
  const bool decayed = kind != kDecayNone;
  const bool elu = a.phi == kPhiElu1;

  __shared__ __align__(16) uint16_t sK[STATE_ONLY ? 8 : C * G::KS];
  __shared__ __align__(16) uint16_t sKT[DK * G::TS];
  __shared__ __align__(16) uint16_t sVT[TV * G::TS];
  __shared__ __align__(16) uint16_t sST[STATE_ONLY ? 8 : 2 * TV * G::KS];
  __shared__ float sB[2][G::CP];

  // Zero the staged tiles once: the padding (dims >= DK, tokens >= C) is
  // never written again and must read as zero in every MFMA.
  {
    uint32_t* z;
    z = reinterpret_cast<uint32_t*>(sKT);
    for (int i = tid; i < DK * G::TS / 2; i += 256) z[i] = 0u;
    z = reinterpret_cast<uint32_t*>(sVT);
    for (int i = tid; i < TV * G::TS / 2; i += 256) z[i] = 0u;
    if constexpr (!STATE_ONLY) {
      z = reinterpret_cast<uint32_t*>(sK);
      for (int i = tid; i < C * G::KS / 2; i += 256) z[i] = 0u;
      z = reinterpret_cast<uint32_t*>(sST);
      for (int i = tid; i < 2 * TV * G::KS / 2; i += 256) z[i] = 0u;
    }
  }

  const size_t head_k = (size_t)bh * L * DK;
  const size_t head_v = (size_t)bh * L * DV;
  const uint16_t* qh = static_cast<const uint16_t*>(a.q) + head_k;
  const uint16_t* kh = static_cast<const uint16_t*>(a.k) + head_k;
  const uint16_t* vh = static_cast<const uint16_t*>(a.v) + head_v + dv0;
  uint16_t* oh = static_cast<uint16_t*>(a.out) + head_v + dv0;
  const float* dtok = (kind == kDecayLog || kind == kDecayGate) ? a.decay + (size_t)bh * L : nullptr;
  const float lg = (kind == kDecayHead) ? logf(a.decay[h]) : 0.0f;

  // ---- initial state of this unit --------------------------------------
  f32x4 accS[G::TPW];
#pragma unroll
  for (int t = 0; t < G::TPW; ++t) accS[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (!STATE_ONLY) {
#pragma unroll
    for (int t = 0; t < G::TPW; ++t) {
      const int tau = wave + 4 * t;
      if (tau < G::NT_S) {
        const int mt = tau / G::NTV, nt = tau % G::NTV;
        const int dv = dv0 + 16 * nt + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dk = 16 * mt + 4 * g4 + i;
          float s = a.state ? a.state[((size_t)bh * DK + dk) * DV + dv] : 0.0f;
          for (int p = 0; p < sigma; ++p) {
            const size_t seg = (size_t)bh * a.P + p;
            s = expf(a.ws_logA[seg]) * s + a.ws_S[(seg * DK + dk) * DV + dv];
          }
          accS[t][i] = s;
        }
        u32x2 w;
        w[0] = pack_bf16x2(accS[t][0], accS[t][1]);
        w[1] = pack_bf16x2(accS[t][2], accS[t][3]);
        *reinterpret_cast<u32x2*>(&sST[(16 * nt + l16) * G::KS + 16 * mt + 4 * g4]) = w;
      }
    }
  }

  // ---- register prefetch of one chunk ----------------------------------
  u32x4 kreg[G::KIT][4];
  u32x4 vreg[G::VIT][4];
  u32x4 qnext[G::SPW][G::KSTEPS];
  u32x4 qcur[G::SPW][G::KSTEPS];
  float dreg0 = 0.0f, dreg1 = 0.0f;
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};

  auto load_chunk = [&](int c) {
    const int t0 = c * C;
#pragma unroll
    for (int it = 0; it < G::KIT; ++it) {
      const int p = tid + 256 * it;
      const int a4 = p / (DK / 8), b8 = p % (DK / 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * a4 + i;
        kreg[it][i] = (p < G::KPIECES && t < L)
                          ? *reinterpret_cast<const u32x4*>(kh + (size_t)t * DK + 8 * b8)
                          : zero4;
      }
    }
#pragma unroll
    for (int it = 0; it < G::VIT; ++it) {
      const int p = tid + 256 * it;
      const int a4 = p / (TV / 8), b8 = p % (TV / 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * a4 + i;
        vreg[it][i] = (p < G::VPIECES && t < L)
                          ? *reinterpret_cast<const u32x4*>(vh + (size_t)t * DV + 8 * b8)
                          : zero4;
      }
    }
    if constexpr (!STATE_ONLY) {
#pragma unroll
      for (int j = 0; j < G::SPW; ++j) {
        const int st = wave + 4 * j;
        const int t = t0 + 16 * st + l16;
#pragma unroll
        for (int s = 0; s < G::KSTEPS; ++s) {
          const int col = 32 * s + 8 * g4;
          qnext[j][s] = (st < G::NSTRIP && t < L && col < DK)
                            ? *reinterpret_cast<const u32x4*>(qh + (size_t)t * DK + col)
                            : zero4;
        }
      }
    }
    if (dtok != nullptr && wave == 0) {
      const int t = t0 + 2 * lane;
      dreg0 = (2 * lane < C && t < L) ? dtok[t] : 0.0f;
      dreg1 = (2 * lane + 1 < C && t + 1 < L) ? dtok[t + 1] : 0.0f;
    }
  };

  float logA = 0.0f;
  load_chunk(c_begin);

  for (int c = c_begin; c < c_end; ++c) {
    const int buf = (c - c_begin) & 1;
    const int t0 = c * C;
    const int nvalid = min(C, L - t0);
    float* sb = sB[buf];

    // (1) in-chunk inclusive prefix of log a (one wave64 scan; padding adds 0)
    if (wave == 0) {
      const int i0 = 2 * lane, i1 = 2 * lane + 1;
      float b0 = 0.0f, b1 = 0.0f;
      if (kind == kDecayHead) {
        b0 = (float)(min(i0, nvalid - 1) + 1) * lg;
        b1 = (float)(min(i1, nvalid - 1) + 1) * lg;
      } else if (decayed) {
        const float x0 = i0 < nvalid ? token_log_decay(kind, dreg0) : 0.0f;
        const float x1 = i1 < nvalid ? token_log_decay(kind, dreg1) : 0.0f;
        float s = x0 + x1;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(s, off, 64);
          if (lane >= off) s += y;
        }
        b0 = s - x1;
        b1 = s;
      }
      if (i0 < G::CP) sb[i0] = b0;
      if (i1 < G::CP) sb[i1] = b1;
    }
    if constexpr (!STATE_ONLY) {
#pragma unroll
      for (int j = 0; j < G::SPW; ++j)
#pragma unroll
        for (int s = 0; s < G::KSTEPS; ++s) {
          u32x4 w = qnext[j][s];
          if (elu) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              w[e] = pack_bf16x2(feature_elu1(bf16_to_f32(w[e] & 0xffffu)),
                                 feature_elu1(bf16_to_f32(w[e] >> 16)));
          }
          qcur[j][s] = w;
        }
    }
    __syncthreads();
    const float bL = sb[G::CP - 1];

    // (2) stage K, K-tilde^T and V^T of this chunk in LDS
#pragma unroll
    for (int it = 0; it < G::KIT; ++it) {
      const int p = tid + 256 * it;
      if (p < G::KPIECES) {
        const int a4 = p / (DK / 8), b8 = p % (DK / 8);
        float kf[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t x = kreg[it][i][w];
            float lo = bf16_to_f32(x & 0xffffu), hi = bf16_to_f32(x >> 16);
            if (elu) { lo = feature_elu1(lo); hi = feature_elu1(hi); }
            kf[i][2 * w] = lo;
            kf[i][2 * w + 1] = hi;
          }
        if constexpr (!STATE_ONLY) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            u32x4 w = kreg[it][i];
            if (elu) {
#pragma unroll
              for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(kf[i][2 * e], kf[i][2 * e + 1]);
            }
            *reinterpret_cast<u32x4*>(&sK[(4 * a4 + i) * G::KS + 8 * b8]) = w;
          }
        }
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = decayed ? __expf(bL - sb[4 * a4 + i]) : 1.0f;
        const int pos = tok_pos(4 * a4);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          u32x2 w;
          w[0] = pack_bf16x2(kf[0][d] * sc[0], kf[1][d] * sc[1]);
          w[1] = pack_bf16x2(kf[2][d] * sc[2], kf[3][d] * sc[3]);
          *reinterpret_cast<u32x2*>(&sKT[(8 * b8 + d) * G::TS + pos]) = w;
        }
      }
    }
#pragma unroll
    for (int it = 0; it < G::VIT; ++it) {
      const int p = tid + 256 * it;
      if (p < G::VPIECES) {
        const int a4 = p / (TV / 8), b8 = p % (TV / 8);
        const int pos = tok_pos(4 * a4);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const int w = d >> 1, sh = (d & 1) * 16;
          u32x2 o;
          o[0] = ((vreg[it][0][w] >> sh) & 0xffffu) | (((vreg[it][1][w] >> sh) & 0xffffu) << 16);
          o[1] = ((vreg[it][2][w] >> sh) & 0xffffu) | (((vreg[it][3][w] >> sh) & 0xffffu) << 16);
          *reinterpret_cast<u32x2*>(&sVT[(8 * b8 + d) * G::TS + pos]) = o;
        }
      }
    }

    // (3) start loading the next chunk while this one computes
    if (c + 1 < c_end) load_chunk(c + 1);
    __syncthreads();

    // (4a) outputs of this chunk's query strips
    if constexpr (!STATE_ONLY) {
      const uint16_t* sSTc = sST + buf * TV * G::KS;
#pragma unroll
      for (int j = 0; j < G::SPW; ++j) {
        const int st = wave + 4 * j;
        if (st < G::NSTRIP) {
          f32x4 pt[G::NSTRIP];
#pragma unroll
          for (int jj = 0; jj < G::NSTRIP; ++jj) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
            if (jj <= st) {
#pragma unroll
              for (int s = 0; s < G::KSTEPS; ++s)
                acc = mfma16x16x32(lds16(&sK[(16 * jj + l16) * G::KS + 32 * s + 8 * g4]),
                                   qcur[j][s], acc);
            }
            pt[jj] = acc;
          }
          // pt[jj][i] = score of query row r against key 16 jj + 4 g4 + i
          const int r = 16 * st + l16;
          const float br = sb[r];
#pragma unroll
          for (int jj = 0; jj < G::NSTRIP; ++jj) {
            if (jj <= st) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int cc = 16 * jj + 4 * g4 + i;
                const float wgt = decayed ? __expf(br - sb[cc]) : 1.0f;
                pt[jj][i] = cc <= r ? pt[jj][i] * wgt : 0.0f;
              }
            }
          }
          u32x4 pb[G::CSTEPS];
#pragma unroll
          for (int s2 = 0; s2 < G::CSTEPS; ++s2) {
            const f32x4 lo = pt[2 * s2];
            const f32x4 hi = (2 * s2 + 1 < G::NSTRIP) ? pt[2 * s2 + 1] : f32x4{0.f, 0.f, 0.f, 0.f};
            pb[s2][0] = pack_bf16x2(lo[0], lo[1]);
            pb[s2][1] = pack_bf16x2(lo[2], lo[3]);
            pb[s2][2] = pack_bf16x2(hi[0], hi[1]);
            pb[s2][3] = pack_bf16x2(hi[2], hi[3]);
          }
          const float erow = decayed ? __expf(br) : 1.0f;
#pragma unroll
          for (int mo = 0; mo < G::NTV; ++mo) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < G::KSTEPS; ++s)
              acc = mfma16x16x32(lds16(&sSTc[(16 * mo + l16) * G::KS + 32 * s + 8 * g4]),
                                 qcur[j][s], acc);
            acc = acc * erow;
#pragma unroll
            for (int s2 = 0; s2 < G::CSTEPS; ++s2) {
              if (2 * s2 <= st)
                acc = mfma16x16x32(lds16(&sVT[(16 * mo + l16) * G::TS + 32 * s2 + 8 * g4]),
                                   pb[s2], acc);
            }
            if (r < nvalid) {
              u32x2 w;
              w[0] = pack_bf16x2(acc[0], acc[1]);
              w[1] = pack_bf16x2(acc[2], acc[3]);
              *reinterpret_cast<u32x2*>(oh + (size_t)(t0 + r) * DV + 16 * mo + 4 * g4) = w;
            }
          }
        }
      }
    }

    // (4b) state update S <- e^{b_last} S + K-tilde^T V
    const bool need_update =
        STATE_ONLY || (c + 1 < c_end) || (sigma == a.P - 1 && a.state != nullptr);
    if (need_update) {
      const float eL = decayed ? __expf(bL) : 1.0f;
      uint16_t* sSTn = sST + (buf ^ 1) * TV * G::KS;
#pragma unroll
      for (int t = 0; t < G::TPW; ++t) {
        const int tau = wave + 4 * t;
        if (tau < G::NT_S) {
          const int mt = tau / G::NTV, nt = tau % G::NTV;
          f32x4 acc = accS[t] * eL;
#pragma unroll
          for (int s2 = 0; s2 < G::CSTEPS; ++s2)
            acc = mfma16x16x32(lds16(&sKT[(16 * mt + l16) * G::TS + 32 * s2 + 8 * g4]),
                               lds16(&sVT[(16 * nt + l16) * G::TS + 32 * s2 + 8 * g4]), acc);
          accS[t] = acc;
          if constexpr (!STATE_ONLY) {
            u32x2 w;
            w[0] = pack_bf16x2(acc[0], acc[1]);
            w[1] = pack_bf16x2(acc[2], acc[3]);
            *reinterpret_cast<u32x2*>(&sSTn[(16 * nt + l16) * G::KS + 16 * mt + 4 * g4]) = w;
          }
        }
      }
    }
    logA += bL;
    __syncthreads();
  }

  // ---- epilogue ---------------------------------------------------------
  float* dst = nullptr;
  if constexpr (STATE_ONLY) {
    dst = a.ws_S + ((size_t)bh * a.P + sigma) * DK * DV;
    if (vt == 0 && tid == 0) a.ws_logA[(size_t)bh * a.P + sigma] = logA;
  } else {
    if (sigma == a.P - 1 && a.state != nullptr) dst = a.state + (size_t)bh * DK * DV;
  }
  if (dst != nullptr) {
#pragma unroll
    for (int t = 0; t < G::TPW; ++t) {
      const int tau = wave + 4 * t;
      if (tau < G::NT_S) {
        const int mt = tau / G::NTV, nt = tau % G::NTV;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[(size_t)(16 * mt + 4 * g4 + i) * DV + dv0 + 16 * nt + l16] = accS[t][i];
      }
    }
  }
}

template <int DK, int TV, int C>
hipError_t launch_one(const ChunkArgs& a, bool state_only, hipStream_t s) {
  const int groups = (a.n_units + 7) / 8;
  const dim3 grid(groups * 8 * a.n_v), block(256);
  if (state_only)
    hipLaunchKernelGGL((chunk_bf16_kernel<DK, TV, C, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((chunk_bf16_kernel<DK, TV, C, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int DK, int TV>
hipError_t dispatch_c(const ChunkArgs& a, bool so, hipStream_t s) {
  switch (a.C) {
    case 16: return launch_one<DK, TV, 16>(a, so, s);
    case 32: return launch_one<DK, TV, 32>(a, so, s);
    case 64: return launch_one<DK, TV, 64>(a, so, s);
    case 128:
      if constexpr (Geo<DK, TV, 128>::LDS_MAIN <= kMaxLds) return launch_one<DK, TV, 128>(a, so, s);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

template <int DK>
hipError_t dispatch_tv(const ChunkArgs& a, bool so, hipStream_t s) {
  switch (a.tv) {
    case 16: return dispatch_c<DK, 16>(a, so, s);
    case 32: return dispatch_c<DK, 32>(a, so, s);
    case 64: return dispatch_c<DK, 64>(a, so, s);
    case 128: return dispatch_c<DK, 128>(a, so, s);
  }
  return hipErrorInvalidValue;
}

template <int DK, int TV>
constexpr size_t lds_of(int C) {
  return C == 16    ? Geo<DK, TV, 16>::LDS_MAIN
         : C == 32  ? Geo<DK, TV, 32>::LDS_MAIN
         : C == 64  ? Geo<DK, TV, 64>::LDS_MAIN
                    : Geo<DK, TV, 128>::LDS_MAIN;
}

template <int DK>
size_t lds_tv(int TV, int C) {
  switch (TV) {
    case 16: return lds_of<DK, 16>(C);
    case 32: return lds_of<DK, 32>(C);
    case 64: return lds_of<DK, 64>(C);
    default: return lds_of<DK, 128>(C);
  }
}

}  // namespace

bool chunk_bf16_supported(int DK, int TV, int C) {
  if (C != 16 && C != 32 && C != 64 && C != 128) return false;
  size_t lds = 0;
  switch (DK) {
    case 16: lds = lds_tv<16>(TV, C); break;
    case 32: lds = lds_tv<32>(TV, C); break;
    case 64: lds = lds_tv<64>(TV, C); break;
    case 128: lds = lds_tv<128>(TV, C); break;
    default: return false;
  }
  return lds <= kMaxLds;
}

hipError_t launch_chunk_bf16(const ChunkArgs& a, bool state_only, hipStream_t s) {
  switch (a.DK) {
    case 16: return dispatch_tv<16>(a, state_only, s);
    case 32: return dispatch_tv<32>(a, state_only, s);
    case 64: return dispatch_tv<64>(a, state_only, s);
    case 128: return dispatch_tv<128>(a, state_only, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace la
