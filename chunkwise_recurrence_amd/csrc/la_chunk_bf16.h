// la_chunk_bf16.h -- chunkwise causal linear attention, bf16 in, gfx950 MFMA.
// Kernel template; one translation unit per key dimension instantiates it.
//
// What one workgroup computes.  A work unit is one head (b, h), one tile of
// TV value columns [dv0, dv0 + TV) and one segment of consecutive chunks of
// the sequence.  For every chunk of C tokens, with b_i the inclusive prefix
// sum of log a over the chunk (every factor below is exp of a value <= 0):
//
//   O_c     = diag(e^b) Q_c S_c + ((Q_c K_c^T) o D_c) V_c,   D_c[i,j] = e^{b_i - b_j} [j <= i]
//   S_{c+1} = e^{b_last} S_c + K_c^T diag(e^{b_last - b}) V_c
//
// This is the chunkwise form of "Linear / Sparse Attention - minimal runnable
// implementation" (linear_attn_chunkwise: inter = Q_c S, intra = masked
// (Q_c K_c^T) V_c, then S += K_c^T V_c, ragged last chunk) with the decay
// folded into S_c and the in-chunk mask, as the linear/sparse attention
// tutorial's section 6.2 says the gated variants do; the per-element decay is
// the log-space construction of CS336 lecture 4 code 1,
// gated_linear_attention_parallel (log D[t,s] = cumsum[t] - cumsum[s]).
//
// Mapping onto gfx950 (4 waves of 64 lanes, v_mfma_f32_16x16x32_bf16):
//   * K and V tiles of a chunk go from HBM straight into LDS with
//     global_load_lds_dwordx4 (no register staging), double-buffered: the
//     next chunk streams in while the current one computes.  Rows are stored
//     with an XOR swizzle of their 16-byte chunks so that 16 lanes reading 16
//     rows at one column hit 16 different bank groups.
//   * K^T and V^T operands (8 consecutive tokens of one key/value column per
//     lane) come from the row-major tiles through ds_read_b64_tr_b16, the
//     LDS transpose read: no transposed copies.
//   * the C query rows of a chunk are split into 16-row strips, strip st
//     belongs to wave st % 4.  A wave computes its strip's scores against key
//     blocks 0..st only (the causal upper blocks are skipped), masks and
//     decays them in fp32 registers, and uses them straight from registers as
//     the B operand of the P.V product: the scores come out of the QK^T MFMA
//     transposed (K is the A operand), which is already the operand layout;
//     the V^T operand reads the matching two runs of 4 tokens.
//   * the state tile S[:, dv0:dv0+TV] lives in fp32 MFMA accumulators, split
//     over the 4 waves by 16x16 tile; after each update a bf16 copy S^T is
//     written to LDS (double-buffered) for the next chunk's inter-chunk term.
//   * Q tiles take the same DMA route into LDS as K (one pipeline stage each)
//     where the LDS holds them at the same pipeline depth: then the loop
//     holds no register loads, whose completion the compiler would wait for
//     by draining every outstanding memory operation (the previous chunk's
//     output stores included) where they cross the loop's back edge.
//     Geometries without room load Q from HBM into B-operand registers.
//   * one workgroup barrier per chunk.
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
#pragma once
#include <type_traits>

#include "la_device.h"

namespace la {
namespace bf16k {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Geometry of one kernel instance: key dim DK, value columns per column group
// TV, chunk C, NG column groups of 4 waves each (the workgroup covers NG*TV
// value columns with 4*NG waves).
template <int DK, int TV, int C, int NG>
struct Geo {
  static constexpr int NW = 4 * NG;                // waves per workgroup
  static constexpr int TVW = NG * TV;              // value columns per workgroup
  static constexpr int CP = C < 32 ? 32 : C;       // chunk padded to whole MFMA k-steps
  static constexpr int KSTEPS = DK < 32 ? 1 : DK / 32;  // k-steps over the key dim
  static constexpr int CSTEPS = CP / 32;           // k-steps over the chunk's tokens
  static constexpr int WCK = DK / 8;               // 16-byte chunks per K row
  static constexpr int WCV = TVW / 8;              // 16-byte chunks per V row (all groups)
  static constexpr int NSTRIP = C / 16;            // 16-row query strips per chunk
  static constexpr int SPW = (NSTRIP + 3) / 4;     // strips per wave
  static constexpr int NTV = TV / 16;              // 16-wide value tiles per group
  static constexpr int NMK = DK / 16;              // 16-wide key tiles
  static constexpr int NT_S = NMK * NTV;           // 16x16 state tiles per group
  static constexpr int TPW = (NT_S + 3) / 4;       // state tiles per wave
  static constexpr int K_TILE = C * DK;            // elements of one K tile
  static constexpr int V_TILE = C * TVW;
  static constexpr int S_TILE = TVW * DK;          // S^T of all groups
  static constexpr int NK_CHUNKS = C * WCK;        // 16-byte chunks of one K tile
  static constexpr int NV_CHUNKS = C * WCV;
  // 1 KB DMA blocks (64 lanes x 16 B) per wave; the last block may be partial
  static constexpr int KBLK = ((NK_CHUNKS + 63) / 64 + NW - 1) / NW;
  static constexpr int VBLK = ((NV_CHUNKS + 63) / 64 + NW - 1) / NW;
  // Every wave issues the same number of memory instructions per chunk (all
  // waves own query strips and equal shares of the K and V tiles): then the
  // wait at the top of a chunk can count instructions and keep later chunks'
  // loads in flight.
  static constexpr bool UNIFORM = NK_CHUNKS % (64 * NW) == 0 && NV_CHUNKS % (64 * NW) == 0 &&
                                  NSTRIP % 4 == 0 && C % NW == 0;
  static constexpr size_t stage_bytes(int n, bool q) {
    return (size_t)n * (2 * (size_t)K_TILE * (q ? 2 : 1) + 2 * (size_t)V_TILE + 4 * (size_t)CP) +
           2 * 2 * (size_t)S_TILE;
  }
  // pipeline depth: three stages (loads two chunks ahead) where they fit
  static constexpr int NSTG = (UNIFORM && stage_bytes(3, false) + 256 <= 160 * 1024) ? 3 : 2;
  // Q tiles copied into LDS with the K and V tiles where that keeps the
  // pipeline depth; otherwise Q goes from HBM into registers.
  static constexpr bool QL = NG == 2 && stage_bytes(NSTG, true) + 256 <= 160 * 1024;
  static constexpr size_t LDS_MAIN = stage_bytes(NSTG, QL) + 256;
  // precomputed per-lane mask/decay weights only while they stay small
  static constexpr bool DM_REGS = NSTRIP <= 4;
  // operands of a whole strip preloaded (more ILP) only in the narrow layout
  static constexpr bool PRELOAD = NG == 1 && NSTRIP <= 4;
};

constexpr size_t kMaxLds = 160 * 1024;

// Byte offset of element (row, col) in a row-major bf16 tile of WC 16-byte
// chunks per row whose chunks are XOR-swizzled by the row's position in its
// 256-byte bank line: 16 consecutive rows read at one logical column land in
// 16 distinct bank groups.
template <int WC>
__device__ __forceinline__ int swz(int row, int col) {
  constexpr int R = WC >= 16 ? 1 : 16 / WC;  // rows per 256-byte bank line
  const int chunk = (col >> 3) ^ ((row / R) & (WC - 1));
  return row * (WC * 16) + (chunk << 4) + ((col & 7) << 1);
}

// An empty volatile statement: the block that holds it runs only when its
// condition holds (the compiler may not if-convert it into always-executed
// arithmetic plus a select).
__device__ __forceinline__ void no_speculation() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ u32x4 lds_b128(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

// Two LDS transpose reads: lane i of each 16-lane group receives column
// (col0 + i) of rows k0a..k0a+3 (elements 0-3) and k0b..k0b+3 (elements 4-7)
// of a swizzled row-major tile; each source lane s addresses row k0 + s/4,
// columns col0 + 4 (s%4) .. +3.
template <int WC>
__device__ __forceinline__ u32x4 lds_tr8(const char* base, int k0a, int k0b, int col0, int l16) {
  const int j = l16 >> 2, m = l16 & 3;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(base + swz<WC>(k0a + j, col0 + 4 * m)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(base + swz<WC>(k0b + j, col0 + 4 * m)));
  u32x4 r;
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  r[0] = a[0];
  r[1] = a[1];
  r[2] = b[0];
  r[3] = b[1];
  return r;
}

__device__ __forceinline__ uint32_t cvt2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// phi = elu + 1 on 8 packed bf16 values.
__device__ __forceinline__ u32x4 elu1_x8(u32x4 w) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = cvt2(feature_elu1(bf16_to_f32(w[e] & 0xffffu)), feature_elu1(bf16_to_f32(w[e] >> 16)));
  return w;
}

// Decay category of a launch (a template parameter, so the kernel has no
// per-element branches on it): none, one constant per head, or per token
// (log a given, or the gate a = exp(-softplus(g)); both arrive as in-chunk
// prefix sums from the prefix pass).
enum { kCatNone = 0, kCatHead = 1, kCatToken = 2 };

// s_waitcnt with only the vector-memory count set (expcnt and lgkmcnt left
// at their maxima): at most n vector memory instructions may be outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int DK, int TV, int C, int NG, int CAT, bool STATE_ONLY>
__global__ __launch_bounds__(256 * NG) void chunk_bf16_kernel(const ChunkArgs a) {
  using G = Geo<DK, TV, C, NG>;
  static_assert(G::NTV <= 4, "a wave's state tiles must share one value tile");
  constexpr int NS = G::NSTG;
  constexpr int NW = G::NW;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < NW);
  const int grp = wave >> 2, wl = wave & 3;  // column group, wave within the group
  const int l16 = lane & 15, g4 = lane >> 4;

  // workgroup -> (unit, value tile); the tiles of one unit share an XCD
  const int f = blockIdx.x;
  const int slot = f >> 3;
  const int vt = slot % a.n_v;
  const int u = (slot / a.n_v) * 8 + (f & 7);
  if (u >= a.n_units) return;
  // state pass: each of the first P - 1 segments in a.sub units of
  // seg_chunks / a.sub chunks; output pass: one unit per segment, composing
  // the sigma * a.sub state units before it
  const int segs = STATE_ONLY ? (a.P - 1) * a.sub : a.P;
  const int bh = u / segs, sigma = u % segs;
  const int span = STATE_ONLY ? a.seg_chunks / a.sub : a.seg_chunks;
  const int nprev = STATE_ONLY ? 0 : sigma * a.sub;
  const size_t unit0 = (size_t)bh * a.P * a.sub;  // this head's first state unit
  const int h = bh % a.H;
  const int dv0 = vt * G::TVW;             // first value column of the workgroup
  const int dvg = dv0 + grp * TV;          // ... of this wave's column group
  const int L = a.L, DV = a.DV;
  const int nchunks = (L + C - 1) / C;
  const int c_begin = sigma * span;
  const int c_end = min(c_begin + span, nchunks);
  constexpr bool decayed = CAT != kCatNone;
  const bool elu = a.phi == kPhiElu1;

  // One array per pipeline stage (not one [NS][...] array): the DMA into one
  // stage and the reads of another are then provably disjoint, so the
  // compiler does not wait for the prefetch before touching LDS.
  constexpr int KB = G::K_TILE * 2, VB = G::V_TILE * 2, BB = CAT == kCatToken ? G::CP : 4;
  __shared__ __align__(16) char sK0[KB], sK1[KB], sK2[NS > 2 ? KB : 16];
  __shared__ __align__(16) char sV0[VB], sV1[VB], sV2[NS > 2 ? VB : 16];
  __shared__ __align__(16) float sB0[BB], sB1[BB], sB2[NS > 2 ? BB : 4];
  constexpr bool QL = G::QL && !STATE_ONLY;
  constexpr int QB = QL ? KB : 16;
  __shared__ __align__(16) char sQ0[QB], sQ1[QB], sQ2[NS > 2 ? QB : 16];
  __shared__ __align__(16) char sST[2][STATE_ONLY ? 16 : G::S_TILE * 2];
  auto stage_k = [&](auto BUF) -> char* {
    constexpr int b = decltype(BUF)::value;
    if constexpr (b == 0) return sK0; else if constexpr (b == 1) return sK1; else return sK2;
  };
  auto stage_v = [&](auto BUF) -> char* {
    constexpr int b = decltype(BUF)::value;
    if constexpr (b == 0) return sV0; else if constexpr (b == 1) return sV1; else return sV2;
  };
  auto stage_q = [&](auto BUF) -> char* {
    constexpr int b = decltype(BUF)::value;
    if constexpr (b == 0) return sQ0; else if constexpr (b == 1) return sQ1; else return sQ2;
  };
  auto stage_b = [&](auto BUF) -> float* {
    constexpr int b = decltype(BUF)::value;
    if constexpr (b == 0) return sB0; else if constexpr (b == 1) return sB1; else return sB2;
  };

  const size_t head_k = (size_t)bh * L * DK;
  const size_t head_v = (size_t)bh * L * DV;
  const uint16_t* qh = static_cast<const uint16_t*>(a.q) + head_k;
  const uint16_t* kh = static_cast<const uint16_t*>(a.k) + head_k;
  const uint16_t* vh = static_cast<const uint16_t*>(a.v) + head_v + dv0;
  uint16_t* og = static_cast<uint16_t*>(a.out) + head_v + dvg;
  const float* bws = CAT == kCatToken ? a.ws_b + (size_t)bh * L : nullptr;
  // per-head decay in log2 units: b_i = (i + 1) lg2 inside a chunk
  const float lg2 = CAT == kCatHead ? log2f(a.decay[h]) : 0.0f;

  // state tiles of this wave: one value tile nt, key tiles mt = (wl + 4 t) / NTV
  const int nt_w = wl % G::NTV;
  // rows of S^T (one per value column of the workgroup) owned by this group start here
  const int srow0 = grp * TV;
  // the 8 tokens of this lane group in state-update k-step s2: k0(s2) + (0..7)
  auto k0_of = [&](int s2) { return (C >= 32) ? 32 * s2 + 8 * g4 : (8 * g4) & 15; };

  // ---- loop-invariant weights (no decay / per-head decay) --------------
  // dm[j][jj][i]: mask and decay of query row r = 16 st + l16 against key
  // c = 16 jj + 4 g4 + i, i.e. [c <= r] gamma^(r - c); er[j] = gamma^(r + 1)
  // (the decay of the carried state seen by row r); vs[s2][e] = gamma^(C-1-t)
  // for the update's tokens t; eLf = gamma^C.  Exponents are all >= 0, so no
  // factor exceeds 1.
  float dm[G::DM_REGS ? G::SPW : 1][G::DM_REGS ? G::NSTRIP : 1][4];
  float er[G::SPW];
  float vs[G::CSTEPS][8];
  float eLf = 1.0f;
  if constexpr (CAT != kCatToken) {
#pragma unroll
    for (int j = 0; j < G::SPW; ++j) {
      const int r = 16 * (wl + 4 * j) + l16;
      er[j] = CAT == kCatHead ? __builtin_amdgcn_exp2f((float)(r + 1) * lg2) : 1.0f;
      if constexpr (G::DM_REGS) {
#pragma unroll
        for (int jj = 0; jj < G::NSTRIP; ++jj)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int cc = 16 * jj + 4 * g4 + i;
            const float w = CAT == kCatHead ? __builtin_amdgcn_exp2f((float)(r - cc) * lg2) : 1.0f;
            dm[j][jj][i] = cc <= r ? w : 0.0f;
          }
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < G::CSTEPS; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vs[s2][e] = CAT == kCatHead
                        ? __builtin_amdgcn_exp2f((float)max(C - 1 - (k0_of(s2) + e), 0) * lg2)
                        : 1.0f;
    if (CAT == kCatHead) eLf = __builtin_amdgcn_exp2f((float)C * lg2);
  }

  // ---- initial state of this unit --------------------------------------
  f32x4 accS[G::TPW];
#pragma unroll
  for (int t = 0; t < G::TPW; ++t) accS[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (!STATE_ONLY) {
    // S_in = S_0 composed with the (decay, increment) pairs of the state
    // units before this segment, four at a time with every load of a batch
    // issued before the first use (one wait for memory per batch).  Units
    // past the last one in the last batch re-read the last one and are
    // weighted out; tiles past a wave's share read tile NT_S - 1 and are
    // never stored.
    const int dv = dvg + 16 * nt_w + l16;
    auto idx_of = [&](int t, int i) {
      const int mt = min(wl + 4 * t, G::NT_S - 1) / G::NTV;
      return (size_t)(16 * mt + 4 * g4 + i) * DV + dv;
    };
    if (a.s0 != nullptr) {
#pragma unroll
      for (int t = 0; t < G::TPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) accS[t][i] = a.s0[(size_t)bh * DK * DV + idx_of(t, i)];
    }
    constexpr int GS = 4;
    for (int p0 = 0; p0 < nprev; p0 += GS) {
      float inc[GS][G::TPW][4], lg[GS];
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        const size_t seg = unit0 + min(p0 + g, nprev - 1);
        lg[g] = a.ws_logA[seg];
#pragma unroll
        for (int t = 0; t < G::TPW; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) inc[g][t][i] = a.ws_S[seg * DK * DV + idx_of(t, i)];
      }
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        // units past the last one are left out by selection (a total decay
        // of -inf times a 0 weight would give NaN)
        const bool m = p0 + g < nprev;
        const float e = exp2f(lg[g]);
#pragma unroll
        for (int t = 0; t < G::TPW; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) accS[t][i] = m ? e * accS[t][i] + inc[g][t][i] : accS[t][i];
      }
    }
#pragma unroll
    for (int t = 0; t < G::TPW; ++t) {
      const int tau = wl + 4 * t;
      if (tau < G::NT_S) {
        const int mt = tau / G::NTV;
        u32x2 w;
        w[0] = cvt2(accS[t][0], accS[t][1]);
        w[1] = cvt2(accS[t][2], accS[t][3]);
        *reinterpret_cast<u32x2*>(&sST[0][swz<G::WCK>(srow0 + 16 * nt_w + l16, 16 * mt + 4 * g4)]) = w;
      }
    }
  } else if (sigma == 0 && a.ws_S0 != nullptr) {
    // the first segment's workgroups copy S_0 for the output pass (its last
    // segment overwrites the caller's state with S_L)
#pragma unroll
    for (int t = 0; t < G::TPW; ++t) {
      const int tau = wl + 4 * t;
      if (tau < G::NT_S) {
        const int mt = tau / G::NTV;
        const int dv = dvg + 16 * nt_w + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const size_t o = ((size_t)bh * DK + 16 * mt + 4 * g4 + i) * DV + dv;
          a.ws_S0[o] = a.state[o];
        }
      }
    }
  }

  // ---- loads of one chunk: K, V tiles and b into LDS, Q into registers ----
  constexpr int KBLK = G::KBLK, VBLK = G::VBLK;
  // per-lane source offsets (elements) of the DMA blocks, relative to the chunk's first row
  int koff[KBLK], krow[KBLK], voff[VBLK], vrow[VBLK];
#pragma unroll
  for (int i = 0; i < KBLK; ++i) {
    const int q = 64 * (wave + NW * i) + lane;
    const int r = q / G::WCK, p = q % G::WCK;
    const int cc = p ^ ((r / (G::WCK >= 16 ? 1 : 16 / G::WCK)) & (G::WCK - 1));
    krow[i] = r;
    koff[i] = r * DK + 8 * cc;
  }
#pragma unroll
  for (int i = 0; i < VBLK; ++i) {
    const int q = 64 * (wave + NW * i) + lane;
    const int r = q / G::WCV, p = q % G::WCV;
    const int cc = p ^ ((r / (G::WCV >= 16 ? 1 : 16 / G::WCV)) & (G::WCV - 1));
    vrow[i] = r;
    voff[i] = r * DV + 8 * cc;
  }
  // Q of each stage, in registers (geometries without Q tiles in LDS)
  u32x4 qst[QL ? 1 : NS][G::SPW][G::KSTEPS];
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};

  // Vector memory instructions one chunk's loads and stores issue per wave
  // (meaningful when G::UNIFORM).
  constexpr int LOADS = KBLK + VBLK + (CAT == kCatToken ? 1 : 0) +
                        (STATE_ONLY ? 0 : QL ? KBLK : G::SPW * G::KSTEPS);
  constexpr int STORES = STATE_ONLY ? 0 : G::SPW * G::NTV;

  auto issue_loads = [&](auto BUF, int c) {
    constexpr int buf = decltype(BUF)::value;
    const int t0 = c * C;
    const bool full = t0 + C <= L;
    const uint16_t* kc = kh + (size_t)t0 * DK;
    const uint16_t* qc = qh + (size_t)t0 * DK;
    const uint16_t* vc = vh + (size_t)t0 * DV;
#pragma unroll
    for (int i = 0; i < KBLK; ++i) {
      const int idx = wave + NW * i;
      const int q = 64 * idx + lane;
      if (64 * idx < G::NK_CHUNKS && q < G::NK_CHUNKS) {
        // rows past the sequence re-read its last row; K rows are zeroed
        // before use, Q rows only give outputs that are not stored
        const int off = full ? koff[i] : koff[i] - (max(krow[i] - (L - 1 - t0), 0)) * DK;
        dma16(kc + off, stage_k(BUF) + 1024 * idx);
        if constexpr (QL) dma16(qc + off, stage_q(BUF) + 1024 * idx);
      }
    }
#pragma unroll
    for (int i = 0; i < VBLK; ++i) {
      const int idx = wave + NW * i;
      const int q = 64 * idx + lane;
      if (64 * idx < G::NV_CHUNKS && q < G::NV_CHUNKS) {
        const int off = full ? voff[i] : voff[i] - (max(vrow[i] - (L - 1 - t0), 0)) * DV;
        dma16(vc + off, stage_v(BUF) + 1024 * idx);
      }
    }
    if constexpr (CAT == kCatToken) {
      // each wave brings its share of the chunk's prefix sums
      constexpr int PER = (C + NW - 1) / NW;
      if (lane < PER && wave * PER + lane < C) {
        const int t = min(t0 + wave * PER + lane, L - 1);
        dma4(bws + t, stage_b(BUF) + wave * PER);
      }
    }
    if constexpr (!STATE_ONLY && !QL) {
#pragma unroll
      for (int j = 0; j < G::SPW; ++j) {
        const int st = wl + 4 * j;
        const int t = t0 + 16 * st + l16;
#pragma unroll
        for (int s = 0; s < G::KSTEPS; ++s) {
          // clamped in-bounds address; rows past the sequence and key columns
          // past DK are zeroed where the registers are used (not here, which
          // would wait for the load)
          const int col = 32 * s + 8 * g4;
          qst[buf][j][s] =
              *reinterpret_cast<const u32x4*>(qh + (size_t)min(t, L - 1) * DK + min(col, DK - 8));
        }
      }
    }
  };

  float logA = 0.0f;

  auto body = [&](auto BUF, int c) {
    constexpr int buf = decltype(BUF)::value;
    const int t0 = c * C;
    const int nvalid = min(C, L - t0);
    char* kb = stage_k(BUF);
    char* vb = stage_v(BUF);
    const float* sb = stage_b(BUF);
    const int sp = (c - c_begin) & 1;  // S^T double buffer: read sp, write sp ^ 1

    // Wait until this wave's loads of chunk c have landed, keeping the loads
    // of later chunks (and the stores issued since) in flight: in issue order,
    // chunk c's loads are followed by nS chunks' stores and nL chunks' loads.
    if constexpr (G::UNIFORM && NS == 3) {
      const int nS = min(NS - 1, c - c_begin), nL = min(NS - 2, c_end - 1 - c);
      if (nS == 2 && nL == 1) wait_vmcnt<2 * STORES + LOADS>();
      else if (nS == 2) wait_vmcnt<2 * STORES>();
      else if (nS == 1 && nL == 1) wait_vmcnt<STORES + LOADS>();
      else if (nS == 1) wait_vmcnt<STORES>();
      else if (nL == 1) wait_vmcnt<LOADS>();
      else wait_vmcnt<0>();
    } else if constexpr (G::UNIFORM) {
      if (c > c_begin) wait_vmcnt<STORES>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    // feature map on this wave's own copies of the chunk's key (and query)
    // blocks, in place: they have landed (the wait above; a copy's lane l
    // fills bytes 16l..16l+15 of its block) and no other wave reads them
    // before the barrier below, which then also publishes the result
    if (elu) {
#pragma unroll
      for (int i = 0; i < KBLK; ++i) {
        const int idx = wave + NW * i;
        const int q = 64 * idx + lane;
        if (64 * idx < G::NK_CHUNKS && q < G::NK_CHUNKS) {
          u32x4* p = reinterpret_cast<u32x4*>(kb + 16 * q);
          *p = elu1_x8(*p);
          if constexpr (QL) {
            u32x4* pq = reinterpret_cast<u32x4*>(stage_q(BUF) + 16 * q);
            *pq = elu1_x8(*pq);
          }
        }
      }
    }
    lds_barrier();  // everybody's loads of chunk c landed; chunk c-1 is finished
    u32x4 qcur[G::SPW][G::KSTEPS];
    if constexpr (!STATE_ONLY) {
      if constexpr (QL) {
        // B operand of the scores: lane (l16, g4) holds query row 16 st + l16,
        // key columns 32 s + 8 g4 .. +7
        const char* qb = stage_q(BUF);
#pragma unroll
        for (int j = 0; j < G::SPW; ++j) {
          const int st = min(wl + 4 * j, G::NSTRIP - 1);
#pragma unroll
          for (int s = 0; s < G::KSTEPS; ++s)
            qcur[j][s] = (DK >= 32 || g4 < 2) ? lds_b128(qb, swz<G::WCK>(16 * st + l16, 32 * s + 8 * g4))
                                              : zero4;
        }
      } else {
#pragma unroll
        for (int j = 0; j < G::SPW; ++j)
#pragma unroll
          for (int s = 0; s < G::KSTEPS; ++s) qcur[j][s] = qst[buf][j][s];
      }
      if (nvalid < C || DK < 32) {
        no_speculation();
#pragma unroll
        for (int j = 0; j < G::SPW; ++j)
#pragma unroll
          for (int s = 0; s < G::KSTEPS; ++s) {
            const bool ok = 16 * (wl + 4 * j) + l16 < nvalid && 32 * s + 8 * g4 < DK;
            qcur[j][s] = ok ? qcur[j][s] : zero4;
          }
      }
      if (!QL && elu) {
        no_speculation();
#pragma unroll
        for (int j = 0; j < G::SPW; ++j)
#pragma unroll
          for (int s = 0; s < G::KSTEPS; ++s) qcur[j][s] = elu1_x8(qcur[j][s]);
      }
    }
    if (c + NS - 1 < c_end) issue_loads(std::integral_constant<int, (buf + NS - 1) % NS>{}, c + NS - 1);

    // a short last chunk: zero the rows past the sequence (they hold clamped copies)
    if (nvalid < C) {
      for (int q = tid; q < (C - nvalid) * G::WCK; q += 64 * NW)
        *reinterpret_cast<u32x4*>(kb + 16 * (nvalid * G::WCK + q)) = zero4;
      for (int q = tid; q < (C - nvalid) * G::WCV; q += 64 * NW)
        *reinterpret_cast<u32x4*>(vb + 16 * (nvalid * G::WCV + q)) = zero4;
      lds_barrier();
    }

    // log2-decay of the chunk's last real token (the state's decay over the chunk)
    float bL = 0.0f;
    if constexpr (CAT == kCatHead) bL = (float)nvalid * lg2;
    if constexpr (CAT == kCatToken) bL = sb[nvalid - 1];

    // (a) outputs of this chunk's query strips.  Every strip computes scores
    // against all key blocks; the causal mask zeroes the blocks past the
    // diagonal.  The slowest wave (the last strip) needs all of them anyway.
    if constexpr (!STATE_ONLY) {
      const char* stc = sST[sp];
#pragma unroll
      for (int j = 0; j < G::SPW; ++j) {
        const int st = wl + 4 * j;
        if (G::NSTRIP >= 4 * (j + 1) || st < G::NSTRIP) {
          f32x4 pt[G::NSTRIP];
#pragma unroll
          for (int jj = 0; jj < G::NSTRIP; ++jj) pt[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
          if constexpr (G::PRELOAD) {
            // all K operands of the strip's scores, then the MFMAs interleaved over key blocks
            u32x4 kA[G::NSTRIP][G::KSTEPS];
#pragma unroll
            for (int jj = 0; jj < G::NSTRIP; ++jj)
#pragma unroll
              for (int s = 0; s < G::KSTEPS; ++s)
                kA[jj][s] = (DK >= 32 || g4 < 2)
                                ? lds_b128(kb, swz<G::WCK>(16 * jj + l16, 32 * s + 8 * g4))
                                : zero4;
#pragma unroll
            for (int s = 0; s < G::KSTEPS; ++s)
#pragma unroll
              for (int jj = 0; jj < G::NSTRIP; ++jj)
                pt[jj] = mfma16x16x32(kA[jj][s], qcur[j][s], pt[jj]);
          } else {
            // one k-step of K operands at a time
#pragma unroll
            for (int s = 0; s < G::KSTEPS; ++s) {
              u32x4 kA[G::NSTRIP];
#pragma unroll
              for (int jj = 0; jj < G::NSTRIP; ++jj)
                kA[jj] = (DK >= 32 || g4 < 2)
                             ? lds_b128(kb, swz<G::WCK>(16 * jj + l16, 32 * s + 8 * g4))
                             : zero4;
#pragma unroll
              for (int jj = 0; jj < G::NSTRIP; ++jj) pt[jj] = mfma16x16x32(kA[jj], qcur[j][s], pt[jj]);
            }
          }
          // pt[jj][i] = score of query row r against key 16 jj + 4 g4 + i: mask and decay
          const int r = 16 * st + l16;
          float erow;
          if constexpr (CAT == kCatToken) {
            const float br = sb[r];
            erow = __builtin_amdgcn_exp2f(br);
#pragma unroll
            for (int jj = 0; jj < G::NSTRIP; ++jj) {
              const f32x4 bc = *reinterpret_cast<const f32x4*>(&sb[16 * jj + 4 * g4]);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int cc = 16 * jj + 4 * g4 + i;
                const float x = pt[jj][i] * __builtin_amdgcn_exp2f(br - bc[i]);
                pt[jj][i] = cc <= r ? x : 0.0f;
              }
            }
          } else if constexpr (G::DM_REGS) {
            erow = er[j];
#pragma unroll
            for (int jj = 0; jj < G::NSTRIP; ++jj)
#pragma unroll
              for (int i = 0; i < 4; ++i) pt[jj][i] *= dm[j][jj][i];
          } else {
            erow = er[j];
#pragma unroll
            for (int jj = 0; jj < G::NSTRIP; ++jj)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int cc = 16 * jj + 4 * g4 + i;
                float x = pt[jj][i];
                if constexpr (CAT == kCatHead) x *= __builtin_amdgcn_exp2f((float)(r - cc) * lg2);
                pt[jj][i] = cc <= r ? x : 0.0f;
              }
          }
          u32x4 pb[G::CSTEPS];
#pragma unroll
          for (int s2 = 0; s2 < G::CSTEPS; ++s2) {
            const f32x4 lo = pt[2 * s2];
            const f32x4 hi = (2 * s2 + 1 < G::NSTRIP) ? pt[2 * s2 + 1] : f32x4{0.f, 0.f, 0.f, 0.f};
            pb[s2][0] = cvt2(lo[0], lo[1]);
            pb[s2][1] = cvt2(lo[2], lo[3]);
            pb[s2][2] = cvt2(hi[0], hi[1]);
            pb[s2][3] = cvt2(hi[2], hi[3]);
          }
          // inter-chunk term (S^T of this group from LDS), then the intra-chunk term
          f32x4 acc[G::NTV];
#pragma unroll
          for (int mo = 0; mo < G::NTV; ++mo) acc[mo] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < G::KSTEPS; ++s) {
            u32x4 sA[G::NTV];
#pragma unroll
            for (int mo = 0; mo < G::NTV; ++mo)
              sA[mo] = (DK >= 32 || g4 < 2)
                           ? lds_b128(stc, swz<G::WCK>(srow0 + 16 * mo + l16, 32 * s + 8 * g4))
                           : zero4;
#pragma unroll
            for (int mo = 0; mo < G::NTV; ++mo) acc[mo] = mfma16x16x32(sA[mo], qcur[j][s], acc[mo]);
          }
          if constexpr (decayed) {
#pragma unroll
            for (int mo = 0; mo < G::NTV; ++mo) acc[mo] = acc[mo] * erow;
          }
#pragma unroll
          for (int s2 = 0; s2 < G::CSTEPS; ++s2) {
            u32x4 vA[G::NTV];
#pragma unroll
            for (int mo = 0; mo < G::NTV; ++mo) {
              if constexpr (C >= 32) {
                // V^T rows for tokens 32 s2 + 4 g4 + (0..3) and 32 s2 + 16 + 4 g4 + (0..3)
                vA[mo] = lds_tr8<G::WCV>(vb, 32 * s2 + 4 * g4, 32 * s2 + 16 + 4 * g4,
                                         srow0 + 16 * mo, l16);
              } else {
                // a 16-token chunk: the second run of 4 tokens lies past the chunk
                const int j2 = l16 >> 2, m2 = l16 & 3;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(vb + swz<G::WCV>(4 * g4 + j2, srow0 + 16 * mo + 4 * m2)));
                const u32x2 lw = __builtin_bit_cast(u32x2, lo);
                vA[mo] = u32x4{lw[0], lw[1], 0u, 0u};
              }
            }
#pragma unroll
            for (int mo = 0; mo < G::NTV; ++mo) acc[mo] = mfma16x16x32(vA[mo], pb[s2], acc[mo]);
          }
          if (r < nvalid) {
#pragma unroll
            for (int mo = 0; mo < G::NTV; ++mo) {
              u32x2 w;
              w[0] = cvt2(acc[mo][0], acc[mo][1]);
              w[1] = cvt2(acc[mo][2], acc[mo][3]);
              *reinterpret_cast<u32x2*>(og + (size_t)(t0 + r) * DV + 16 * mo + 4 * g4) = w;
            }
          }
        }
      }
    }

    // (b) state update S <- e^{b_last} S + K^T diag(e^{b_last - b}) V.  The
    // transpose reads take every lane of the wave (they exchange data within
    // each 16-lane group); for a 16-token chunk the lane groups past the chunk
    // read rows 0..15 again and are zeroed afterwards.
    if (G::TPW > 1 || wl < G::NT_S) {
      char* stn = sST[sp ^ 1];
      u32x4 vB[G::CSTEPS];
#pragma unroll
      for (int s2 = 0; s2 < G::CSTEPS; ++s2) {
        const int k0 = k0_of(s2);
        u32x4 w = lds_tr8<G::WCV>(vb, k0, k0 + 4, srow0 + 16 * nt_w, l16);
        if constexpr (decayed) {
          float sc[8];
          if constexpr (CAT == kCatToken) {
            const f32x4 b0 = *reinterpret_cast<const f32x4*>(&sb[k0]);
            const f32x4 b1 = *reinterpret_cast<const f32x4*>(&sb[k0 + 4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sc[e] = __builtin_amdgcn_exp2f(bL - b0[e]);
              sc[4 + e] = __builtin_amdgcn_exp2f(bL - b1[e]);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) sc[e] = vs[s2][e];
            if (nvalid < C) {  // the short last chunk decays from its last real token
              no_speculation();
#pragma unroll
              for (int e = 0; e < 8; ++e)
                sc[e] = __builtin_amdgcn_exp2f((float)max(nvalid - 1 - (k0 + e), 0) * lg2);
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)  // word e holds tokens k0 + 2e, k0 + 2e + 1
            w[e] = cvt2(bf16_to_f32(w[e] & 0xffffu) * sc[2 * e], bf16_to_f32(w[e] >> 16) * sc[2 * e + 1]);
        }
        vB[s2] = (C < 32 && g4 >= 2) ? zero4 : w;
      }
      if constexpr (decayed) {
        float eL = eLf;
        if (CAT == kCatToken || nvalid < C) {
          no_speculation();
          eL = __builtin_amdgcn_exp2f(bL);
        }
#pragma unroll
        for (int t = 0; t < G::TPW; ++t) accS[t] = accS[t] * eL;
      }
      if constexpr (G::PRELOAD) {
        u32x4 kA2[G::TPW][G::CSTEPS];
#pragma unroll
        for (int t = 0; t < G::TPW; ++t) {
          const int mt = min((wl + 4 * t) / G::NTV, G::NMK - 1);
#pragma unroll
          for (int s2 = 0; s2 < G::CSTEPS; ++s2) {
            const int k0 = k0_of(s2);
            const u32x4 w = lds_tr8<G::WCK>(kb, k0, k0 + 4, 16 * mt, l16);
            kA2[t][s2] = (C < 32 && g4 >= 2) ? zero4 : w;
          }
        }
#pragma unroll
        for (int s2 = 0; s2 < G::CSTEPS; ++s2)
#pragma unroll
          for (int t = 0; t < G::TPW; ++t) accS[t] = mfma16x16x32(kA2[t][s2], vB[s2], accS[t]);
      } else {
#pragma unroll
        for (int t = 0; t < G::TPW; ++t) {
          const int mt = min((wl + 4 * t) / G::NTV, G::NMK - 1);
#pragma unroll
          for (int s2 = 0; s2 < G::CSTEPS; ++s2) {
            const int k0 = k0_of(s2);
            u32x4 w = lds_tr8<G::WCK>(kb, k0, k0 + 4, 16 * mt, l16);
            w = (C < 32 && g4 >= 2) ? zero4 : w;
            accS[t] = mfma16x16x32(w, vB[s2], accS[t]);
          }
        }
      }
      if constexpr (!STATE_ONLY) {
#pragma unroll
        for (int t = 0; t < G::TPW; ++t) {
          const int tau = wl + 4 * t;
          if (tau < G::NT_S) {
            const int mt = tau / G::NTV;
            u32x2 w;
            w[0] = cvt2(accS[t][0], accS[t][1]);
            w[1] = cvt2(accS[t][2], accS[t][3]);
            *reinterpret_cast<u32x2*>(&stn[swz<G::WCK>(srow0 + 16 * nt_w + l16, 16 * mt + 4 * g4)]) = w;
          }
        }
      }
    }
    logA += bL;
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  issue_loads(S0{}, c_begin);
  if constexpr (NS == 3) {
    if (c_begin + 1 < c_end) issue_loads(S1{}, c_begin + 1);
    for (int c = c_begin; c < c_end; c += 3) {
      body(S0{}, c);
      if (c + 1 < c_end) body(S1{}, c + 1);
      if (c + 2 < c_end) body(S2{}, c + 2);
    }
  } else {
    for (int c = c_begin; c < c_end; c += 2) {
      body(S0{}, c);
      if (c + 1 < c_end) body(S1{}, c + 1);
    }
  }

  // ---- epilogue ---------------------------------------------------------
  float* dst = nullptr;
  if constexpr (STATE_ONLY) {
    dst = a.ws_S + (unit0 + sigma) * DK * DV;
    if (vt == 0 && tid == 0) a.ws_logA[unit0 + sigma] = logA;
  } else {
    if (sigma == a.P - 1 && a.state != nullptr) dst = a.state + (size_t)bh * DK * DV;
  }
  if (dst != nullptr) {
#pragma unroll
    for (int t = 0; t < G::TPW; ++t) {
      const int tau = wl + 4 * t;
      if (tau < G::NT_S) {
        const int mt = tau / G::NTV;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[(size_t)(16 * mt + 4 * g4 + i) * DV + dvg + 16 * nt_w + l16] = accS[t][i];
      }
    }
  }
}

// ---- launch and dispatch ----------------------------------------------------
template <int DK, int TV, int C, int NG, int CAT>
hipError_t launch_one(const ChunkArgs& a, bool state_only, hipStream_t s) {
  const int groups = (a.n_units + 7) / 8;
  const dim3 grid(groups * 8 * a.n_v), block(256 * NG);
  if (state_only)
    hipLaunchKernelGGL((chunk_bf16_kernel<DK, TV, C, NG, CAT, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((chunk_bf16_kernel<DK, TV, C, NG, CAT, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int DK, int TV, int NG, int CAT>
hipError_t dispatch_c(const ChunkArgs& a, bool so, hipStream_t s) {
  switch (a.C) {
    case 16:
      if constexpr (Geo<DK, TV, 16, NG>::LDS_MAIN <= kMaxLds) return launch_one<DK, TV, 16, NG, CAT>(a, so, s);
      return hipErrorInvalidValue;
    case 32:
      if constexpr (Geo<DK, TV, 32, NG>::LDS_MAIN <= kMaxLds) return launch_one<DK, TV, 32, NG, CAT>(a, so, s);
      return hipErrorInvalidValue;
    case 64:
      if constexpr (Geo<DK, TV, 64, NG>::LDS_MAIN <= kMaxLds) return launch_one<DK, TV, 64, NG, CAT>(a, so, s);
      return hipErrorInvalidValue;
    case 128:
      if constexpr (Geo<DK, TV, 128, NG>::LDS_MAIN <= kMaxLds) return launch_one<DK, TV, 128, NG, CAT>(a, so, s);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

// a.tv is the width of one column group; a.ng the number of groups (1 or 2)
template <int DK, int CAT>
hipError_t dispatch_tv(const ChunkArgs& a, bool so, hipStream_t s) {
  if (a.ng == 2) {
    switch (a.tv) {
      case 16: return dispatch_c<DK, 16, 2, CAT>(a, so, s);
      case 32: return dispatch_c<DK, 32, 2, CAT>(a, so, s);
      case 64: return dispatch_c<DK, 64, 2, CAT>(a, so, s);
    }
    return hipErrorInvalidValue;
  }
  switch (a.tv) {
    case 16: return dispatch_c<DK, 16, 1, CAT>(a, so, s);
    case 32: return dispatch_c<DK, 32, 1, CAT>(a, so, s);
    case 64: return dispatch_c<DK, 64, 1, CAT>(a, so, s);
  }
  return hipErrorInvalidValue;
}

template <int DK>
hipError_t dispatch_cat(const ChunkArgs& a, bool so, hipStream_t s) {
  switch (a.decay_kind) {
    case kDecayNone: return dispatch_tv<DK, kCatNone>(a, so, s);
    case kDecayHead: return dispatch_tv<DK, kCatHead>(a, so, s);
    default: return dispatch_tv<DK, kCatToken>(a, so, s);
  }
}

template <int DK, int TV, int NG>
constexpr size_t lds_of(int C) {
  return C == 16    ? Geo<DK, TV, 16, NG>::LDS_MAIN
         : C == 32  ? Geo<DK, TV, 32, NG>::LDS_MAIN
         : C == 64  ? Geo<DK, TV, 64, NG>::LDS_MAIN
                    : Geo<DK, TV, 128, NG>::LDS_MAIN;
}

template <int DK>
constexpr size_t lds_tv(int TV, int NG, int C) {
  return NG == 2 ? (TV == 16 ? lds_of<DK, 16, 2>(C) : TV == 32 ? lds_of<DK, 32, 2>(C) : lds_of<DK, 64, 2>(C))
                 : (TV == 16 ? lds_of<DK, 16, 1>(C) : TV == 32 ? lds_of<DK, 32, 1>(C) : lds_of<DK, 64, 1>(C));
}

}  // namespace bf16k

// One per key dimension, each in its own translation unit.
hipError_t launch_chunk_bf16_dk16(const ChunkArgs& a, bool state_only, hipStream_t s);
hipError_t launch_chunk_bf16_dk32(const ChunkArgs& a, bool state_only, hipStream_t s);
hipError_t launch_chunk_bf16_dk64(const ChunkArgs& a, bool state_only, hipStream_t s);
hipError_t launch_chunk_bf16_dk128(const ChunkArgs& a, bool state_only, hipStream_t s);

}  // namespace la
