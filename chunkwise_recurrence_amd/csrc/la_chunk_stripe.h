// la_chunk_stripe.h -- chunkwise causal linear attention, bf16 in, gfx950
// v_mfma_f32_32x32x16_bf16; each wave owns a 32-column stripe of the value
// dimension and keeps its part of the state in registers.
//
// The arithmetic is the same as the per-strip kernel's (la_chunk_bf16.h): for
// every chunk of C tokens, with b the inclusive in-chunk prefix of log a,
//
//   O_c     = diag(e^b) Q_c S_c + ((Q_c K_c^T) o D_c) V_c,   D_c[i,j] = e^{b_i - b_j} [j <= i]
//   S_{c+1} = e^{b_last} S_c + K_c^T diag(e^{b_last - b}) V_c
//
// (the chunkwise form of "Linear / Sparse Attention - minimal runnable
// implementation", linear_attn_chunkwise, with the decay folded into S_c and
// the in-chunk mask as the linear/sparse attention tutorial's section 6.2
// says; the per-element decay is the log-space construction of CS336 lecture 4
// code 1, gated_linear_attention_parallel).  Only the work split differs:
//
//   * a workgroup of NWV waves owns one head, NWV*32 value columns and one
//     segment of the sequence; wave w owns value columns [32w, 32w + 32).
//   * S[:, stripe] (d_k x 32, fp32) lives in the wave's MFMA accumulators as
//     d_k/32 tiles of 32x32.  The inter-chunk term is computed transposed,
//     O^T[stripe, rows] = S^T Q^T, with the accumulators themselves (packed to
//     bf16) as the A operand: an accumulator lane holds one value column and
//     the keys {8q + 4h + (0..3)}, so the A operand's k positions run over
//     keys 16s + 4h + (0..3) and 16s + 8 + 4h + (0..3), and the Q^T operand
//     reads the same keys (two 8-byte LDS reads).  S never goes through LDS.
//   * the causal 32x32 score blocks P^T[J, I] = K_J Q_I^T (J <= I) are spread
//     over the waves, masked and decayed in registers and written to LDS as
//     bf16 P~ (row-major, swizzled); after one barrier every wave reads the
//     rows it needs as the B operand of O^T += V^T P~^T.
//   * V^T operands (lane = value column, 8 consecutive tokens) come from the
//     row-major V tile through ds_read_b64_tr_b16; the same registers, scaled
//     by e^{b_last - b_t}, are the B operand of the state update
//     S += K^T diag(e^{b_last - b}) V, whose K^T operand is read the same way.
//   * Q, K, V tiles stream from HBM into LDS with global_load_lds_dwordx4,
//     NSTG chunks deep; workgroup barriers wait for LDS only, so the prefetch
//     stays in flight across them.
//   * an output row block (32 rows x 32 columns) is transposed back through a
//     2 KB LDS slot of its wave and leaves as 16-byte stores, 64 contiguous
//     bytes per row.
//
// NORM adds the normalised form (the tutorial's section 2.2, boxed
// recurrence): z_t = a_t z_{t-1} + phi(k_t) is carried like one more value
// column of ones and o_t = phi(q_t)^T S_t / phi(q_t)^T z_t.  Per chunk the
// denominator is e^{b_i} phi(q_i).z_c (v_dot2_f32_bf16 over the inter term's
// q operand pairs against z rounded to bf16 pairs, each row block on a stripe
// other than 0) plus the row sums of the masked, decayed scores (taken where
// the score blocks are made); z itself is updated by the waves of stripe 0
// from the K^T operands and token weights of the state update.
//
// The per-channel decay (CAT kCatChannel; GLA's diagonal gate, the tutorial's
// section 2.4: S_t = diag(a_t) S_{t-1} + k_t v_t^T with a_t a vector over the
// key channels) no longer factors out of the contraction over keys:
// P[i][j] = sum_d q_id k_jd e^{b_id - b_jd}, with b[t][d] the in-chunk prefix
// of log a per channel.  The factor is split around r_d = b_{last,d} / 2,
//
//   q~_id = q_id e^{b_id - r_d},   k~_jd = k_jd e^{r_d - b_jd}
//
// (each exponent within half the chunk's total decay), which turns the scores
// into q~ k~^T, the inter-chunk term into q~ (diag(e^r) S) and the update into
// S' = diag(e^{b_last - r}) (diag(e^r) S + k~^T V).  The prefix runs over
// log a loaded straight into registers (each wave scans its own key channels
// over the whole chunk: a thread takes a run of tokens of four or two
// channels, and the runs combine by lane shifts inside a 16-lane row, with no
// exchange between waves), and q~, k~ replace q, k in their LDS tiles, so
// everything after is the kernel's usual MFMA work.
// The split stays in range while every channel's log2 decay over a chunk sums
// to at least -kSplitMax (factors up to 2^96).  A workgroup that meets a chunk
// beyond that flags itself, and a second launch (EXACT) recomputes exactly the
// flagged workgroups' segments -- the secondary-chunking idea for GLA's gate,
// taken to single tokens: scores per element in fp32 with each exponent a
// direct sum of log2 a over (j, i] (never a difference of prefix sums), the
// inter term against q^ = q e^{b} and the update S' = diag(e^{b_last}) S +
// (k e^{b_last - b})^T V, every exponent <= 0.  The state pass always uses
// that exact update, so its segment increments are right whatever the decay.
//
// STATE_ONLY computes a segment's state increment and total log2 decay from a
// zero state (the first pass of the segment split).  It walks the segment's
// chunks last to first, weighting token t by e^{B_end - B_t} directly (the sum
// does not depend on the order), so the chunks it reads last -- the starts of
// the segments -- are the ones the output pass reads first, while they may
// still sit in the memory-side cache.  (With the per-channel decay it walks
// forward and applies the exact update above.)
// The main pass composes
// the exclusive prefix of the (decay, state) pairs in its prologue, the
// parallel / associative scan idea of the tutorial's section 3.3.
#pragma once
#include <type_traits>

#include "la_device.h"

namespace la {
namespace stripe {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr size_t kMaxLds = 160 * 1024;

// SO: the state-only pass, which stages no Q tile and needs no P~, partial
// exchange or output staging (so it can prefetch deeper).  CH: the
// per-channel decay, whose log a tile goes to registers (TPR tokens of CPT
// channels per thread) instead of per-wave token weights to LDS.
template <int DK, int NWV, int KH, int C, bool SO = false, bool CH = false>
struct Geo {
  static constexpr int NW = NWV * KH;           // waves of the workgroup
  static constexpr int TVW = 32 * NWV;          // value columns of the workgroup
  static constexpr int WCK = DK / 8;            // 16-byte chunks per Q/K row
  static constexpr int WCV = TVW / 8;           // ... per V row
  static constexpr int WCP = C / 8;             // ... per P~ row
  static constexpr int NRB = C / 32;            // 32-row blocks of a chunk
  static constexpr int NKS = DK / 16;           // 16-key MFMA steps
  static constexpr int NMK = DK / 32;           // 32-key state tiles
  static constexpr int NKS_OWN = NKS / KH;      // ... of one wave's key part
  static constexpr int NMK_OWN = NMK / KH;
  static constexpr int NTS = C / 16;            // 16-token MFMA steps
  static constexpr int NB = NRB * (NRB + 1) / 2;  // causal 32x32 score blocks
  static constexpr int BPW = (NB + NW - 1) / NW;  // score blocks per wave (at most)
  static constexpr int RBW = (NRB + KH - 1) / KH;  // output row blocks per wave (at most)
  static constexpr int QK_BYTES = C * DK * 2;
  static constexpr int V_BYTES = C * TVW * 2;
  static constexpr int QK_BLK = QK_BYTES / 1024;  // 1 KB DMA blocks (64 lanes x 16 B)
  static constexpr int V_BLK = V_BYTES / 1024;
  static constexpr int QK_PER = (QK_BLK + NW - 1) / NW;  // per wave
  static constexpr int V_PER = (V_BLK + NW - 1) / NW;
  // per-channel decay: wave w scans key channels CPW w .. CPW w + CPW - 1
  // over the whole chunk.  Its lanes are CPW / CPT channel groups of CPT
  // channels (four -- one 16-byte load per token -- unless that takes more
  // than 16 runs, else two) times R runs of TPR consecutive tokens; a group's
  // runs are R consecutive lanes of one 16-lane row
  static constexpr int CPW = DK / NW;
  static constexpr int CPT = (CPW % 4 == 0 && 256 / CPW <= 16) ? 4 : 2;
  static constexpr int R = 64 * CPT / CPW;
  static constexpr int TPR = R >= 1 && C % R == 0 ? C / R : 0;
  // vector memory instructions of one chunk per wave (at most)
  static constexpr int LOADS_MAX = (SO ? 1 : 2) * QK_PER + V_PER + (CH ? TPR : 1);
  static constexpr int STORES = SO ? 0 : 2 * RBW;
  // every wave issues the same memory instructions per chunk and their count
  // fits the 6-bit vmcnt, so the wait at the top of a chunk can count them
  static constexpr bool UNIFORM = QK_BLK % NW == 0 && V_BLK % NW == 0 && NRB % KH == 0 &&
                                  STORES + LOADS_MAX < 64;
  static constexpr size_t XCH_BYTES = KH > 1 ? (size_t)NWV * NRB * 4096 : 16;
  // the key parts' exchange, or (per-channel decay, output pass) the exact
  // path's log2 a tile [C][DK] fp32, which it holds before the exchange is used
  static constexpr size_t LA_BYTES = (CH && !SO) ? 4 * (size_t)C * DK : 16;
  static constexpr size_t XU_BYTES = XCH_BYTES > LA_BYTES ? XCH_BYTES : LA_BYTES;
  // the normalised form's z, denominator partials and row sums (counted for
  // every instance, so both forms run the same pipeline depth)
  static constexpr size_t NORM_BYTES = 2 * 4 * (size_t)DK + 4 * (size_t)C * (KH + NRB);
  // per-wave token weights, or (per-channel decay) the per-channel factors
  // e^r, e^{b_last - r}
  static constexpr size_t W_BYTES = CH ? 2 * 4 * (size_t)DK
                                       : 2 * 4 * (size_t)NW * C;
  static constexpr size_t stage_bytes(int n) {
    return SO ? (size_t)n * ((size_t)QK_BYTES + (size_t)V_BYTES + 4 * (size_t)C) +
                    W_BYTES + NORM_BYTES + 256
              : (size_t)n * (2 * (size_t)QK_BYTES + (size_t)V_BYTES + 4 * (size_t)C) +
                    2 * (size_t)C * C + W_BYTES + XU_BYTES + 2048 * (size_t)NW  + NORM_BYTES + 256;
  }
  // the per-channel decay's prefetch registers stay bounded (at most 32 values
  // per thread and stage)
  static constexpr bool CH_OK = !CH || (R <= 16 && TPR >= 1 && TPR * CPT <= 32 && DK >= 32);
  static constexpr int NSTG =
      (UNIFORM && stage_bytes(3) <= kMaxLds && 2 * STORES + LOADS_MAX < 64) ? 3 : 2;
  static constexpr size_t LDS = stage_bytes(NSTG);
  static_assert(QK_BYTES % 1024 == 0 && V_BYTES % 1024 == 0, "tiles are whole DMA blocks");
  static_assert(KH == 1 || NMK % KH == 0, "key parts hold whole 32-key tiles");
};

// Row-major bf16 tiles with WC 16-byte chunks per row keep their chunks
// XOR-swizzled by g(m), m = the row's 256-byte bank line.  g is a bijection on
// m mod WC, so 16 consecutive rows read at one logical chunk hit 16 distinct
// bank slots; and 4 consecutive rows move an aligned group of 4 chunks to 4
// distinct groups, so a transpose read (4 rows x 4 chunks per 32 lanes) is
// conflict-free too.
template <int WC>
__device__ __forceinline__ int swz_xor(int row) {
  constexpr int RPL = WC >= 16 ? 1 : 16 / WC;   // rows per bank line
  constexpr int A = WC >= 4 ? WC / 4 : 1;       // groups of 4 chunks per row
  const int m = row / RPL;
  return (((m & (A - 1)) << 2) | ((m / A) & 3)) & (WC - 1);
}
template <int WC>
__device__ __forceinline__ int swz(int row, int col) {
  const int chunk = (col >> 3) ^ swz_xor<WC>(row);
  return row * (WC * 16) + (chunk << 4) + ((col & 7) << 1);
}

__device__ __forceinline__ u32x4 lds_b128(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ u32x2 lds_b64(const char* base, int off) {
  return *reinterpret_cast<const u32x2*>(base + off);
}

// Transpose read of 8 tokens of one column: lane i of each 16-lane group gets
// column col0 + i of rows k0 .. k0+3 (elements 0-3) and k0+4 .. k0+7 (4-7).
// Every lane of the wave must take part.
template <int WC>
__device__ __forceinline__ u32x4 lds_tr8(const char* base, int k0, int col0, int l16) {
  const int j = l16 >> 2, m = l16 & 3;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(base + swz<WC>(k0 + j, col0 + 4 * m)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(base + swz<WC>(k0 + 4 + j, col0 + 4 * m)));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return u32x4{a[0], a[1], b[0], b[1]};
}

__device__ __forceinline__ uint32_t cvt2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// c + a.lo * b.lo + a.hi * b.hi over two packed bf16 values (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 elu1_x8(u32x4 w) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = cvt2(feature_elu1(bf16_to_f32(w[e] & 0xffffu)), feature_elu1(bf16_to_f32(w[e] >> 16)));
  return w;
}

__device__ __forceinline__ void no_speculation() { asm volatile("" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for data exchanged through LDS: this wave's LDS accesses
// complete, then s_barrier; no memory fence, so global loads in flight stay
// in flight.  The empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS writes of this wave complete before its later LDS reads of other lanes'
// data (LDS requests of one wave are processed in order; this only stops the
// compiler from reordering).
__device__ __forceinline__ void lds_wave_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  asm volatile("" ::: "memory");
}

enum { kCatNone = 0, kCatHead = 1, kCatToken = 2, kCatChannel = 3 };

// Over a group of R lanes (R <= 16 consecutive lanes of a 16-lane row,
// r = lane % R): the sum of x over the group's lanes below r (prefix) or
// above r (suffix) -- a Hillis-Steele scan of the group shifted by one lane;
// its step d only matters when d < R - 1, the first lane's shifted value
// being 0
template <int R>
__device__ __forceinline__ float group_excl_prefix(float x, int r) {
  const float x1 = dpp_row_shr<1>(x);
  float s = r >= 1 ? x1 : 0.0f;
  if constexpr (R > 2) { const float y = dpp_row_shr<1>(s); if (r >= 1) s += y; }
  if constexpr (R > 3) { const float y = dpp_row_shr<2>(s); if (r >= 2) s += y; }
  if constexpr (R > 5) { const float y = dpp_row_shr<4>(s); if (r >= 4) s += y; }
  if constexpr (R > 9) { const float y = dpp_row_shr<8>(s); if (r >= 8) s += y; }
  return s;
}
template <int R>
__device__ __forceinline__ float group_excl_suffix(float x, int r) {
  const float x1 = dpp_row_shl<1>(x);
  float s = r + 1 < R ? x1 : 0.0f;
  if constexpr (R > 2) { const float y = dpp_row_shl<1>(s); if (r + 1 < R) s += y; }
  if constexpr (R > 3) { const float y = dpp_row_shl<2>(s); if (r + 2 < R) s += y; }
  if constexpr (R > 5) { const float y = dpp_row_shl<4>(s); if (r + 4 < R) s += y; }
  if constexpr (R > 9) { const float y = dpp_row_shl<8>(s); if (r + 8 < R) s += y; }
  return s;
}

// N (2 or 4) consecutive bf16 of an LDS tile, 4N-byte aligned, to fp32 and back
template <int N>
__device__ __forceinline__ void lds_bf16_get(const char* p, float* f) {
  if constexpr (N == 4) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    f[0] = bf16_to_f32(w[0] & 0xffffu);
    f[1] = bf16_to_f32(w[0] >> 16);
    f[2] = bf16_to_f32(w[1] & 0xffffu);
    f[3] = bf16_to_f32(w[1] >> 16);
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    f[0] = bf16_to_f32(w & 0xffffu);
    f[1] = bf16_to_f32(w >> 16);
  }
}
template <int N>
__device__ __forceinline__ void lds_bf16_put(char* p, const float* f) {
  if constexpr (N == 4) {
    u32x2 w;
    w[0] = cvt2(f[0], f[1]);
    w[1] = cvt2(f[2], f[3]);
    *reinterpret_cast<u32x2*>(p) = w;
  } else {
    *reinterpret_cast<uint32_t*>(p) = cvt2(f[0], f[1]);
  }
}

// Per-channel decay: the largest |log2 decay| of a chunk (per channel) the
// split q e^{b - r}, k e^{r - b} takes (factors up to 2^96); beyond it the
// chunk takes the exact path.
constexpr float kSplitMax = 192.0f;

// (I, J) of causal score block b in the order (0,0), (1,0), (1,1), (2,0), ...
__host__ __device__ constexpr int block_i(int b) {
  int i = 0;
  while ((i + 1) * (i + 2) / 2 <= b) ++i;
  return i;
}
__host__ __device__ constexpr int block_j(int b) { return b - block_i(b) * (block_i(b) + 1) / 2; }

// Per-channel decay, exact path: P~[i][j] = sum_d phi(q)_id phi(k)_jd 2^{D_ijd}
// for j <= i < nvalid (zero elsewhere), with D_ijd the sum of log2 a over
// tokens j+1 .. i of channel d, accumulated directly as j steps down: no
// difference of prefix sums (no cancellation, no inf - inf) and every
// exponent <= 0.  GR lanes share a query row, CPG channels each; the q and k
// tiles (row-major bf16, swizzled) hold phi already, lat is the chunk's log2 a
// [C][DK] fp32 and sP the bf16 P~ tile.
template <int DK, int C, int NW>
__device__ __forceinline__ void exact_scores(const char* qb, const char* kb,
                                                        const float* lat, char* sP, int nvalid,
                                                        int tid) {
  constexpr int WCK = DK / 8, WCP = C / 8;
  constexpr int T = 64 * NW;
  constexpr int GR0 = T >= 8 * C ? 8 : T >= 4 * C ? 4 : T >= 2 * C ? 2 : 1;
  constexpr int GR = GR0 < DK / 8 ? GR0 : DK / 8;
  constexpr int CPG = DK / GR;
  for (int task = tid; task < C * GR; task += T) {
    const int i = task / GR, g = task % GR, c0 = CPG * g;
    float qv[CPG], D[CPG];
#pragma unroll
    for (int m = 0; m < CPG / 8; ++m) {
      const u32x4 w = lds_b128(qb, swz<WCK>(i, c0 + 8 * m));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[8 * m + 2 * e] = bf16_to_f32(w[e] & 0xffffu);
        qv[8 * m + 2 * e + 1] = bf16_to_f32(w[e] >> 16);
      }
    }
#pragma unroll
    for (int c = 0; c < CPG; ++c) D[c] = 0.0f;
    const int jtop = i < nvalid ? i : -1;
    for (int j = jtop; j >= 0; --j) {
      float p = 0.0f;
#pragma unroll
      for (int m = 0; m < CPG / 8; ++m) {
        const u32x4 w = lds_b128(kb, swz<WCK>(j, c0 + 8 * m));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p += qv[8 * m + 2 * e] * bf16_to_f32(w[e] & 0xffffu) *
               __builtin_amdgcn_exp2f(D[8 * m + 2 * e]);
          p += qv[8 * m + 2 * e + 1] * bf16_to_f32(w[e] >> 16) *
               __builtin_amdgcn_exp2f(D[8 * m + 2 * e + 1]);
        }
      }
#pragma unroll
      for (int sh = 1; sh < GR; sh <<= 1) p += __shfl_xor(p, sh);
      if (j % GR == g) *reinterpret_cast<uint16_t*>(sP + swz<WCP>(i, j)) = (uint16_t)cvt2(p, 0.0f);
#pragma unroll
      for (int m = 0; m < CPG / 4; ++m) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(&lat[j * DK + c0 + 4 * m]);
#pragma unroll
        for (int e = 0; e < 4; ++e) D[4 * m + e] += x[e];
      }
    }
    for (int j = jtop + 1; j < C; ++j)
      if (j % GR == g) *reinterpret_cast<uint16_t*>(sP + swz<WCP>(i, j)) = 0;
  }
}

template <int DK, int NWV, int KH, int C, int CAT, bool STATE_ONLY, bool NORM, bool EXACT = false>
__global__ __launch_bounds__(64 * NWV * KH) void chunk_stripe_kernel(const ChunkArgs a) {
  constexpr bool CHN = CAT == kCatChannel;
  static_assert(!EXACT || (CHN && !STATE_ONLY), "the exact pass is the per-channel output pass");
  // per-channel decay: whether every chunk takes the exact form (the state
  // pass, and the exact re-run of flagged output-pass workgroups)
  constexpr bool XF = CHN && (STATE_ONLY || EXACT);
  static_assert(!(CHN && NORM), "the normalised form takes no per-channel decay");
  using G = Geo<DK, NWV, KH, C, STATE_ONLY, CHN>;
  static_assert(G::CH_OK, "per-channel decay layout");
  constexpr int NS = G::NSTG;
  constexpr int NW = G::NW;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < NW);
  const int l32 = lane & 31, h = lane >> 5, l16 = lane & 15, g4 = lane >> 4;
  // wave = stripe + NWV * key part: the wave owns value columns
  // [32 stripe, +32) of the tile and keys [part * DK / KH, +DK / KH) of the state
  const int stripe = wave % NWV, part = wave / NWV;

  // workgroup -> (unit, value tile); the tiles of one unit share an XCD
  const int f = blockIdx.x;
  const int slot = f >> 3;
  const int vt = slot % a.n_v;
  const int u = (slot / a.n_v) * 8 + (f & 7);
  if (u >= a.n_units) return;
  // the exact re-run recomputes only the workgroups the fast pass flagged
  if constexpr (EXACT)
    if (a.ws_flag[f] == 0) return;
  // state pass: each of the first P - 1 segments in a.sub units of
  // seg_chunks / a.sub chunks; output pass: one unit per segment, composing
  // the sigma * a.sub state units before it
  const int segs = STATE_ONLY ? (a.P - 1) * a.sub : a.P;
  const int bh = u / segs, sigma = u % segs;
  const int span = STATE_ONLY ? a.seg_chunks / a.sub : a.seg_chunks;
  const int nprev = STATE_ONLY ? 0 : sigma * a.sub;
  const size_t unit0 = (size_t)bh * a.P * a.sub;  // this head's first state unit
  const int hd = bh % a.H;
  const int L = a.L, DV = a.DV;
  const int dv0 = vt * G::TVW;      // first value column of the workgroup
  const int cw = 32 * stripe;       // first column of this wave's stripe, in the tile
  const int mk0 = part * G::NMK_OWN;  // first 32-key state tile of this wave
  const int nchunks = (L + C - 1) / C;
  const int c_begin = sigma * span;
  const int c_end = min(c_begin + span, nchunks);
  const bool elu = a.phi == kPhiElu1;

  __shared__ __align__(16) char sQ0[STATE_ONLY ? 16 : G::QK_BYTES], sQ1[STATE_ONLY ? 16 : G::QK_BYTES],
      sQ2[(NS > 2 && !STATE_ONLY) ? G::QK_BYTES : 16];
  __shared__ __align__(16) char sK0[G::QK_BYTES], sK1[G::QK_BYTES], sK2[NS > 2 ? G::QK_BYTES : 16];
  __shared__ __align__(16) char sV0[G::V_BYTES], sV1[G::V_BYTES], sV2[NS > 2 ? G::V_BYTES : 16];
  __shared__ __align__(16) float sB0[CAT == kCatToken ? C : 4], sB1[CAT == kCatToken ? C : 4],
      sB2[(NS > 2 && CAT == kCatToken) ? C : 4];
  __shared__ __align__(16) char sP[STATE_ONLY ? 16 : 2 * C * C];
  // partial inter-chunk terms handed between the key parts of a stripe:
  // [stripe][row block][16-byte chunk k][lane]
  // (per-channel decay: the exact path's log2 a tile [C][DK] shares it; it is
  // written and read before the exchange)
  __shared__ __align__(16) char sX[STATE_ONLY ? 16 : G::XU_BYTES];
  // per-channel decay, fast output pass: set when a chunk's decay is too strong
  // for the split (the workgroup's results are then recomputed exactly)
  __shared__ int sBad;
  // per-wave weights of the current chunk: [0] e^{b_last - b_t}, [1] e^{b_t}
  __shared__ __align__(16) float sW[CHN ? 1 : NW][2][CHN ? 4 : C];
  // per-channel decay: e^r and e^{b_last - r} per key channel
  __shared__ __align__(16) float sER[CHN ? DK : 4], sEL[CHN ? DK : 4];
  // normalised form: z (double-buffered by chunk parity), the denominators'
  // inter-chunk partials per key part and the score row sums per key block
  __shared__ __align__(16) float sZ[NORM ? 2 : 1][NORM ? DK : 4];
  __shared__ __align__(16) float sDen[(NORM && !STATE_ONLY) ? KH : 1][(NORM && !STATE_ONLY) ? C : 4];
  __shared__ __align__(16) float sRS[(NORM && !STATE_ONLY) ? G::NRB : 1][(NORM && !STATE_ONLY) ? C : 4];
  // per-wave staging of one bf16 output row block: 32 rows x 64 bytes
  __shared__ __align__(16) char sO[STATE_ONLY ? 1 : NW][STATE_ONLY ? 16 : 2048];

  auto stage_q = [&](auto BUF) -> char* {
    constexpr int b = decltype(BUF)::value;
    if constexpr (b == 0) return sQ0; else if constexpr (b == 1) return sQ1; else return sQ2;
  };
  auto stage_k = [&](auto BUF) -> char* {
    constexpr int b = decltype(BUF)::value;
    if constexpr (b == 0) return sK0; else if constexpr (b == 1) return sK1; else return sK2;
  };
  auto stage_v = [&](auto BUF) -> char* {
    constexpr int b = decltype(BUF)::value;
    if constexpr (b == 0) return sV0; else if constexpr (b == 1) return sV1; else return sV2;
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
  uint16_t* oh = static_cast<uint16_t*>(a.out) + head_v + dv0 + cw;
  const float* bws = CAT == kCatToken ? a.ws_b + (size_t)bh * L : nullptr;
  const float lg2 = CAT == kCatHead ? log2f(a.decay[hd]) : 0.0f;  // b_i = (i + 1) lg2
  float* wq = sW[CHN ? 0 : wave][0];
  float* eq = sW[CHN ? 0 : wave][1];
  // per-channel decay: this thread's run of tokens and its key channels
  // ch0 .. ch0 + CPT - 1
  const float* dch = CHN ? a.decay + (size_t)bh * L * DK : nullptr;
  const int run = CHN ? lane % G::R : 0;
  const int ch0 = CHN ? G::CPW * wave + G::CPT * (lane / G::R) : 0;

  // ---- loop-invariant mask/decay weights of this wave's score blocks ------
  // block (I, J), register r: query row i = 32 I + l32, token
  // j = 32 J + 8 (r / 4) + 4 h + r % 4; weight [j <= i] gamma^(i - j).
  float dm[(CAT == kCatToken || CHN) ? 1 : G::BPW][16];
  if constexpr (CAT != kCatToken && !CHN && !STATE_ONLY) {
#pragma unroll
    for (int bb = 0; bb < G::BPW; ++bb) {
      const int b = wave + NW * bb;
      const int I = b < G::NB ? block_i(b) : 0, J = b < G::NB ? block_j(b) : 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * I + l32, j = 32 * J + 8 * (r >> 2) + 4 * h + (r & 3);
        const float w = CAT == kCatHead ? __builtin_amdgcn_exp2f((float)(i - j) * lg2) : 1.0f;
        dm[bb][r] = j <= i ? w : 0.0f;
      }
    }
  }

  // ---- initial state of this wave's part ---------------------------------
  // own tile t (state tile mk0 + t), register r: key 32 (mk0 + t) + 8 (r / 4)
  // + 4 h + r % 4, value column dv0 + cw + l32
  f32x16 accS[G::NMK_OWN];
#pragma unroll
  for (int t = 0; t < G::NMK_OWN; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) accS[t][r] = 0.0f;
  if constexpr (!STATE_ONLY) {
    // S_in = S_0 composed with the (decay, increment) pairs of the state
    // units before this segment, GS at a time with every load of a batch
    // issued before the first use: one wait for memory per batch, not one per
    // unit and state element.  Units past the last one in the last batch
    // re-read the last one and are weighted out (factor 1, increment 0).
    const int dv = dv0 + cw + l32;
    auto dk_of = [&](int t, int r) { return 32 * (mk0 + t) + 8 * (r >> 2) + 4 * h + (r & 3); };
    if (a.s0 != nullptr) {
#pragma unroll
      for (int t = 0; t < G::NMK_OWN; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) accS[t][r] = a.s0[((size_t)bh * DK + dk_of(t, r)) * DV + dv];
    }
    constexpr int GS = CHN ? 2 : 4;
    for (int p0 = 0; p0 < nprev; p0 += GS) {
      float inc[GS][G::NMK_OWN][16], lg[GS][CHN ? G::NMK_OWN : 1][CHN ? 16 : 1];
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        const size_t seg = unit0 + min(p0 + g, nprev - 1);
#pragma unroll
        for (int t = 0; t < G::NMK_OWN; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            inc[g][t][r] = a.ws_S[(seg * DK + dk_of(t, r)) * DV + dv];
            if constexpr (CHN) lg[g][t][r] = a.ws_logA[seg * DK + dk_of(t, r)];
          }
        if constexpr (!CHN) lg[g][0][0] = a.ws_logA[seg];
      }
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        // units past the last one are left out by selection (a total decay
        // of -inf times a 0 weight would give NaN)
        const bool m = p0 + g < nprev;
#pragma unroll
        for (int t = 0; t < G::NMK_OWN; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float la2 = CHN ? lg[g][CHN ? t : 0][CHN ? r : 0] : lg[g][0][0];
            accS[t][r] = m ? exp2f(la2) * accS[t][r] + inc[g][t][r] : accS[t][r];
          }
      }
    }
  }
  // State pass: the first segment's workgroups copy S_0 for the output pass,
  // whose last segment overwrites the caller's state with S_L.  The values are
  // loaded here, ahead of the first tile loads, and stored after the last
  // chunk, so the copy adds no latency of its own.
  const bool copy_s0 = STATE_ONLY && sigma == 0 && a.ws_S0 != nullptr;
  auto s0_index = [&](int t, int r) -> size_t {
    return ((size_t)bh * DK + 32 * (mk0 + t) + 8 * (r >> 2) + 4 * h + (r & 3)) * DV + dv0 + cw + l32;
  };
  float s0v[STATE_ONLY ? G::NMK_OWN : 1][16];
  if constexpr (STATE_ONLY) {
    if (copy_s0) {
#pragma unroll
      for (int t = 0; t < G::NMK_OWN; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) s0v[t][r] = a.state[s0_index(t, r)];
    }
  }
  // normalised form: the waves of stripe 0 hold z for their keys, lane l32
  // of own tile t holding key 32 (mk0 + t) + l32
  float zr[NORM ? G::NMK_OWN : 1];
  if constexpr (NORM) {
#pragma unroll
    for (int t = 0; t < G::NMK_OWN; ++t) {
      const int dk = 32 * (mk0 + t) + l32;
      float zv = 0.0f;
      if constexpr (!STATE_ONLY) {
        // composed like S_in: four segments' loads per wait
        zv = a.z0 ? a.z0[(size_t)bh * DK + dk] : 0.0f;
        for (int p0 = 0; p0 < nprev; p0 += 4) {
          float zi[4], lz[4];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const size_t seg = unit0 + min(p0 + g, nprev - 1);
            lz[g] = a.ws_logA[seg];
            zi[g] = a.ws_z[seg * DK + dk];
          }
#pragma unroll
          for (int g = 0; g < 4; ++g) zv = p0 + g < nprev ? exp2f(lz[g]) * zv + zi[g] : zv;
        }
      }
      zr[t] = zv;
      if (stripe == 0 && h == 0) sZ[0][dk] = zv;
    }
  }

  // bf16 A operands of the inter-chunk term: own key step s (global step
  // part * NKS_OWN + s) uses own tile s / 2, registers 8 (s % 2) .. +7
  u32x4 sbf[G::NKS_OWN];
  // normalised form: the stripe that forms row block I's phi(q).z partials
  // (never stripe 0 when there are others)
  auto dz_stripe = [](int I) { return NWV == 1 ? 0 : 1 + I % (NWV - 1); };
  auto pack_state = [&]() {
#pragma unroll
    for (int s = 0; s < G::NKS_OWN; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sbf[s][e] = cvt2(accS[s >> 1][8 * (s & 1) + 2 * e], accS[s >> 1][8 * (s & 1) + 2 * e + 1]);
  };

  // ---- loads of one chunk: Q, K, V tiles and b into LDS --------------------
  // DMA block i of a tile covers its 16-byte chunks 64 i .. 64 i + 63 (in
  // swizzled order); lane l moves chunk 64 i + l.  Per-lane source offsets:
  int koff[G::QK_PER], krow[G::QK_PER], voff[G::V_PER], vrow[G::V_PER];
#pragma unroll
  for (int i = 0; i < G::QK_PER; ++i) {
    const int p = 64 * (wave + NW * i) + lane;
    const int r = p / G::WCK, pc = p % G::WCK;
    const int cc = pc ^ swz_xor<G::WCK>(r);
    krow[i] = r;
    koff[i] = r * DK + 8 * cc;
  }
#pragma unroll
  for (int i = 0; i < G::V_PER; ++i) {
    const int p = 64 * (wave + NW * i) + lane;
    const int r = p / G::WCV, pc = p % G::WCV;
    const int cc = pc ^ swz_xor<G::WCV>(r);
    vrow[i] = r;
    voff[i] = r * DV + 8 * cc;
  }
  constexpr int LOADS = (STATE_ONLY ? 1 : 2) * G::QK_PER + G::V_PER + (CAT == kCatToken ? 1 : 0) +
                        (CHN ? G::TPR : 0);
  constexpr int STORES = STATE_ONLY ? 0 : G::STORES;

  // iteration it handles chunk chunk_of(it): forward in the output pass,
  // backward in the state pass (forward with the per-channel decay)
  const int n_it = c_end - c_begin;
  auto chunk_of = [&](int it) { return (STATE_ONLY && !CHN) ? c_end - 1 - it : c_begin + it; };

  // per-channel decay: log a of this thread's tokens and channels, per stage
  typedef float fcv __attribute__((ext_vector_type(G::CPT)));
  // (the fast output pass with two stages reads a chunk's registers before
  // the next chunk's loads are issued into them, so one set serves; the exact
  // form reads them again after the issue)
  constexpr int LB = (CHN && !XF && NS == 2) ? 1 : (CHN ? NS : 1);
  fcv lreg[LB][CHN ? G::TPR : 1];

  auto issue_loads = [&](auto BUF, int it) {
    const int c = chunk_of(it);
    const int t0 = c * C;
    const bool full = t0 + C <= L;
    const uint16_t* kc = kh + (size_t)t0 * DK;
    const uint16_t* qc = qh + (size_t)t0 * DK;
    const uint16_t* vc = vh + (size_t)t0 * DV;
#pragma unroll
    for (int i = 0; i < G::QK_PER; ++i) {
      const int idx = wave + NW * i;
      if (idx < G::QK_BLK) {
        // rows past the sequence re-read its last row; they are zeroed before use
        const int off = full ? koff[i] : koff[i] - max(krow[i] - (L - 1 - t0), 0) * DK;
        // (the output pass reads q, k and v for the last time)
        if constexpr (STATE_ONLY) {
          dma16(kc + off, stage_k(BUF) + 1024 * idx);
        } else {
          dma16_nt(kc + off, stage_k(BUF) + 1024 * idx);
          dma16_nt(qc + off, stage_q(BUF) + 1024 * idx);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < G::V_PER; ++i) {
      const int idx = wave + NW * i;
      if (idx < G::V_BLK) {
        const int off = full ? voff[i] : voff[i] - max(vrow[i] - (L - 1 - t0), 0) * DV;
        if constexpr (STATE_ONLY) dma16(vc + off, stage_v(BUF) + 1024 * idx);
        else dma16_nt(vc + off, stage_v(BUF) + 1024 * idx);
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
    if constexpr (CHN) {
      // rows past the sequence re-read its last row; they are zeroed before use
      constexpr int buf = decltype(BUF)::value;
#pragma unroll
      for (int i = 0; i < G::TPR; ++i) {
        const int t = min(t0 + run * G::TPR + i, L - 1);
        lreg[buf % LB][i] = *reinterpret_cast<const fcv*>(dch + (size_t)t * DK + ch0);
      }
    }
  };

  if (CHN && tid == 0) sBad = 0;

  float logA = 0.0f;
  fcv logAc = fcv{};  // per-channel decay: totals of this thread's channels
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};

  auto body = [&](auto BUF, int it) {
    constexpr int buf = decltype(BUF)::value;
    const int c = chunk_of(it);
    const int t0 = c * C;
    const int nvalid = min(C, L - t0);
    char* qb = stage_q(BUF);
    char* kb = stage_k(BUF);
    char* vb = stage_v(BUF);
    const float* sb = stage_b(BUF);

    // Wait until this wave's loads of iteration it have landed, keeping later
    // iterations' loads (and the stores issued since) in flight: in issue
    // order, its loads are followed by nS iterations' stores and nL
    // iterations' loads.
    if constexpr (G::UNIFORM && NS == 3) {
      const int nS = min(NS - 1, it), nL = min(NS - 2, n_it - 1 - it);
      if (nS == 2 && nL == 1) wait_vmcnt<2 * STORES + LOADS>();
      else if (nS == 2) wait_vmcnt<2 * STORES>();
      else if (nS == 1 && nL == 1) wait_vmcnt<STORES + LOADS>();
      else if (nS == 1) wait_vmcnt<STORES>();
      else if (nL == 1) wait_vmcnt<LOADS>();
      else wait_vmcnt<0>();
    } else if constexpr (G::UNIFORM) {
      if (it > 0) wait_vmcnt<STORES>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    // feature map on this wave's own copies of the chunk's key (and query)
    // blocks, in place: they have landed (the wait above; a copy's lane l
    // fills bytes 16l..16l+15 of its block) and no other wave reads them
    // before the barrier below, which then also publishes the result (the
    // per-channel decay applies the map in its rescaling pass instead)
    if (elu && !CHN) {
#pragma unroll
      for (int i = 0; i < G::QK_PER; ++i) {
        const int idx = wave + NW * i;
        if (idx < G::QK_BLK) {
          u32x4* p = reinterpret_cast<u32x4*>(kb + 1024 * idx + 16 * lane);
          *p = elu1_x8(*p);
          if constexpr (!STATE_ONLY) {
            u32x4* pq = reinterpret_cast<u32x4*>(qb + 1024 * idx + 16 * lane);
            *pq = elu1_x8(*pq);
          }
        }
      }
    }
    lds_barrier();  // everybody's loads of this chunk landed; the previous one is finished
    // per-channel decay: this thread's in-run prefix of log2 a (tokens past the
    // sequence contribute nothing), taken from its registers before the next
    // chunk's loads are issued -- the compiler waits for those registers by
    // count and does not see the tile copies, so a later wait would also
    // hold back the next chunk's copies
    constexpr float kLog2e = 1.4426950408889634f;
    fcv bl[CHN ? G::TPR : 1];
    fcv accb = fcv{};
    if constexpr (CHN) {
#pragma unroll
      for (int i = 0; i < G::TPR; ++i) {
        const fcv x = lreg[buf % LB][i] * kLog2e;
        accb += run * G::TPR + i < nvalid ? x : fcv{};
        bl[i] = accb;
      }
      // the run total depends on every register: using it here keeps the
      // compiler's wait for them ahead of the copies below
#pragma unroll
      for (int e = 0; e < G::CPT; ++e) asm volatile("" ::"v"(accb[e]));
    }
    if (it + NS - 1 < n_it) issue_loads(std::integral_constant<int, (buf + NS - 1) % NS>{}, it + NS - 1);

    // a short last chunk: zero the rows past the sequence (clamped copies)
    if (nvalid < C) {
      for (int q = tid; q < (C - nvalid) * G::WCK; q += 64 * NW) {
        *reinterpret_cast<u32x4*>(kb + 16 * (nvalid * G::WCK + q)) = zero4;
        if constexpr (!STATE_ONLY) *reinterpret_cast<u32x4*>(qb + 16 * (nvalid * G::WCK + q)) = zero4;
      }
      for (int q = tid; q < (C - nvalid) * G::WCV; q += 64 * NW)
        *reinterpret_cast<u32x4*>(vb + 16 * (nvalid * G::WCV + q)) = zero4;
      lds_barrier();
    }

    if constexpr (CHN) {
      // the run totals' exclusive prefix (off) and suffix (later) over the
      // group's runs by row shifts (sums only, so log a = -inf stays -inf),
      // and the group's total from its last run
      fcv off, tot, later = fcv{};
#pragma unroll
      for (int e = 0; e < G::CPT; ++e) {
        off[e] = group_excl_prefix<G::R>(accb[e], run);
        // (a group of 16 is a whole row: DPP row_share reads its last lane)
        if constexpr (G::R == 16)
          tot[e] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                 0, __builtin_bit_cast(int, off[e] + accb[e]),
                                                 0x150 + 15, 0xf, 0xf, false));
        else
          tot[e] = __shfl(off[e] + accb[e], lane | (G::R - 1));
        if constexpr (XF) later[e] = group_excl_suffix<G::R>(accb[e], run);
      }
      if constexpr (!XF) {
        // the split below puts factors up to 2^{-tot/2} into q and k: a chunk
        // whose log2 decay sums below -kSplitMax in any channel (or is not a
        // number) flags the workgroup for the exact re-run
        bool in_range = true;
#pragma unroll
        for (int e = 0; e < G::CPT; ++e) in_range = in_range && tot[e] >= -kSplitMax;
        if (!in_range) sBad = 1;
        const fcv rr = tot * 0.5f;  // r = b_last / 2
        // q~ = phi(q) e^{b - r}, k~ = phi(k) e^{r - b}, in place
        // (every read of the thread's q, k elements is issued before the
        // first write back, so the reads' LDS latency overlaps; d = b - r, with
        // the k factor 2^-d through v_exp_f32's negate modifier)
        auto rescale = [&](auto ELU) {
          const fcv c0 = off - rr;
          float kf[G::TPR][G::CPT], qf[G::TPR][G::CPT];
#pragma unroll
          for (int i = 0; i < G::TPR; ++i) {
            const int o = swz<G::WCK>(run * G::TPR + i, ch0);
            lds_bf16_get<G::CPT>(kb + o, kf[i]);
            lds_bf16_get<G::CPT>(qb + o, qf[i]);
          }
#pragma unroll
          for (int i = 0; i < G::TPR; ++i) {
            const fcv d = bl[i] + c0;
#pragma unroll
            for (int e = 0; e < G::CPT; ++e) {
              if constexpr (decltype(ELU)::value) {
                kf[i][e] = feature_elu1(kf[i][e]);
                qf[i][e] = feature_elu1(qf[i][e]);
              }
              kf[i][e] *= __builtin_amdgcn_exp2f(-d[e]);
              qf[i][e] *= __builtin_amdgcn_exp2f(d[e]);
            }
          }
#pragma unroll
          for (int i = 0; i < G::TPR; ++i) {
            const int o = swz<G::WCK>(run * G::TPR + i, ch0);
            lds_bf16_put<G::CPT>(kb + o, kf[i]);
            lds_bf16_put<G::CPT>(qb + o, qf[i]);
          }
        };
        if (elu) rescale(std::true_type{});
        else rescale(std::false_type{});
        if (run == 0) {
          fcv er, el;
#pragma unroll
          for (int e = 0; e < G::CPT; ++e) {
            er[e] = __builtin_amdgcn_exp2f(rr[e]);
            el[e] = __builtin_amdgcn_exp2f(tot[e] - rr[e]);
          }
          *reinterpret_cast<fcv*>(&sER[ch0]) = er;
          *reinterpret_cast<fcv*>(&sEL[ch0]) = el;
        }
      } else {
        // exact form: every factor is 2^(a direct sum of log2 a <= 0).  sf[i]:
        // the sum over the run's tokens after token i (exclusive suffix)
        fcv sf[G::TPR];
        fcv acs = fcv{};
#pragma unroll
        for (int i = G::TPR - 1; i >= 0; --i) {
          sf[i] = acs;
          acs += run * G::TPR + i < nvalid ? lreg[buf % LB][i] * kLog2e : fcv{};
        }
        if constexpr (!STATE_ONLY) {
          // phi on this thread's q and k elements in place, its log2 a into the tile
          float* lat = reinterpret_cast<float*>(sX);
#pragma unroll
          for (int i = 0; i < G::TPR; ++i) {
            const int t = run * G::TPR + i;
            const int o = swz<G::WCK>(t, ch0);
            if (elu) {
              float kf[G::CPT], qf[G::CPT];
              lds_bf16_get<G::CPT>(kb + o, kf);
              lds_bf16_get<G::CPT>(qb + o, qf);
#pragma unroll
              for (int e = 0; e < G::CPT; ++e) {
                kf[e] = feature_elu1(kf[e]);
                qf[e] = feature_elu1(qf[e]);
              }
              lds_bf16_put<G::CPT>(kb + o, kf);
              lds_bf16_put<G::CPT>(qb + o, qf);
            }
            *reinterpret_cast<fcv*>(&lat[t * DK + ch0]) =
                t < nvalid ? lreg[buf % LB][i] * kLog2e : fcv{};
          }
          lds_barrier();
          exact_scores<DK, C, NW>(qb, kb, reinterpret_cast<const float*>(sX), sP, nvalid, tid);
          lds_barrier();  // the scores have read the tiles the rescaling below overwrites
        }
        // q^ = phi(q) e^{b}, k^ = phi(k) e^{b_last - b}, in place (the state
        // pass maps k here; the flag is tested once, not per element)
        // (reads first, as above)
        auto rescale = [&](auto ELU) {
          float kf[G::TPR][G::CPT], qf[STATE_ONLY ? 1 : G::TPR][G::CPT];
#pragma unroll
          for (int i = 0; i < G::TPR; ++i) {
            const int o = swz<G::WCK>(run * G::TPR + i, ch0);
            lds_bf16_get<G::CPT>(kb + o, kf[i]);
            if constexpr (!STATE_ONLY) lds_bf16_get<G::CPT>(qb + o, qf[i]);
          }
#pragma unroll
          for (int i = 0; i < G::TPR; ++i) {
            const fcv ek = sf[i] + later;
#pragma unroll
            for (int e = 0; e < G::CPT; ++e) {
              if constexpr (STATE_ONLY && decltype(ELU)::value) kf[i][e] = feature_elu1(kf[i][e]);
              kf[i][e] *= __builtin_amdgcn_exp2f(ek[e]);
            }
            if constexpr (!STATE_ONLY) {
              const fcv eb = off + bl[i];
#pragma unroll
              for (int e = 0; e < G::CPT; ++e) qf[i][e] *= __builtin_amdgcn_exp2f(eb[e]);
            }
          }
#pragma unroll
          for (int i = 0; i < G::TPR; ++i) {
            const int o = swz<G::WCK>(run * G::TPR + i, ch0);
            lds_bf16_put<G::CPT>(kb + o, kf[i]);
            if constexpr (!STATE_ONLY) lds_bf16_put<G::CPT>(qb + o, qf[i]);
          }
        };
        if (STATE_ONLY && elu) rescale(std::true_type{});
        else rescale(std::false_type{});
        if (run == 0) {
          fcv er, el;
#pragma unroll
          for (int e = 0; e < G::CPT; ++e) {
            er[e] = 1.0f;
            el[e] = __builtin_amdgcn_exp2f(tot[e]);
          }
          *reinterpret_cast<fcv*>(&sER[ch0]) = er;
          *reinterpret_cast<fcv*>(&sEL[ch0]) = el;
        }
      }
      logAc += tot;
      lds_barrier();
    }
    // rows of this wave's state tiles scaled by a per-channel factor from LDS
    // (register r of own tile t holds key 32 (mk0 + t) + 8 (r / 4) + 4 h + r % 4)
    auto scale_rows = [&](const float* f) {
#pragma unroll
      for (int t = 0; t < G::NMK_OWN; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&f[32 * (mk0 + t) + 8 * q + 4 * h]);
#pragma unroll
          for (int e = 0; e < 4; ++e) accS[t][4 * q + e] *= x[e];
        }
    };

    // log2 decay of the chunk's last real token
    float bL = 0.0f;
    if constexpr (CAT == kCatHead) bL = (float)nvalid * lg2;
    if constexpr (CAT == kCatToken) bL = sb[nvalid - 1];

    // per-token weights of this wave: e^{b_last - b_t} (update; 0 past the
    // chunk) and e^{b_t} (inter-chunk term), t = lane (+ 64).  The state pass
    // folds in the decay of the chunks after this one (logA so far).
    if constexpr (CAT != kCatNone && !CHN) {
      const float wofs = STATE_ONLY ? logA + bL : bL;
#pragma unroll
      for (int t = lane; t < C; t += 64) {
        const float bt = CAT == kCatHead ? (float)(t + 1) * lg2 : sb[t];
        wq[t] = t < nvalid ? __builtin_amdgcn_exp2f(wofs - bt) : 0.0f;
        if constexpr (!STATE_ONLY) eq[t] = __builtin_amdgcn_exp2f(bt);
      }
      lds_wave_sync();
    }

    // V^T operands of this wave's stripe: lane (value cw + l32, h), tokens
    // 16 ks + 8 h + (0..7)
    u32x4 vA[G::NTS];
#pragma unroll
    for (int ks = 0; ks < G::NTS; ++ks)
      vA[ks] = lds_tr8<G::WCV>(vb, 16 * ks + 8 * (g4 >> 1), cw + 16 * (g4 & 1), l16);

    // (3) state update of this wave's tiles (after the outputs; it reads only
    // K, V and the weights, and S_c is already packed for the inter term)
    auto state_update = [&]() {
      // S <- e^{b_last} S + K^T diag(e^{b_last - b}) V
      // (state pass: S <- S + K^T diag(e^{B_end - B}) V)
      // (per-channel decay: S <- diag(e^{b_last - r}) (diag(e^r) S + k~^T V))
      // (per-channel decay, exact form -- the state pass, and the output
      // pass's exact path: S <- diag(e^{b_last}) S + k^^T V)
      if constexpr (XF) scale_rows(sEL);
      if constexpr (CAT != kCatNone && !CHN && !STATE_ONLY) {
        const float eL = __builtin_amdgcn_exp2f(bL);
#pragma unroll
        for (int t = 0; t < G::NMK_OWN; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) accS[t][r] *= eL;
      }
      float zacc[NORM ? G::NMK_OWN : 1];
      if constexpr (NORM) {
#pragma unroll
        for (int t = 0; t < G::NMK_OWN; ++t) zacc[t] = 0.0f;
      }
#pragma unroll
      for (int ks = 0; ks < G::NTS; ++ks) {
        u32x4 vB = vA[ks];
        float w[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
        if constexpr (CAT == kCatNone && NORM) {
          // rows past a short last chunk are zeroed after the feature map;
          // the mask keeps them out of z whatever they hold
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = 16 * ks + 8 * h + e < nvalid ? 1.0f : 0.0f;
        }
        if constexpr (CAT != kCatNone && !CHN) {
          const int tb = 16 * ks + 8 * h;
          const f32x4 w0 = *reinterpret_cast<const f32x4*>(&wq[tb]);
          const f32x4 w1 = *reinterpret_cast<const f32x4*>(&wq[tb + 4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            w[e] = w0[e];
            w[4 + e] = w1[e];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
            vB[e] = cvt2(bf16_to_f32(vB[e] & 0xffffu) * w[2 * e], bf16_to_f32(vB[e] >> 16) * w[2 * e + 1]);
        }
        // the token weights as packed bf16 pairs for z (the value operand
        // carries them in bf16 too)
        uint32_t wp[NORM ? 4 : 1];
        if constexpr (NORM) {
#pragma unroll
          for (int e = 0; e < 4; ++e) wp[e] = cvt2(w[2 * e], w[2 * e + 1]);
        }
#pragma unroll
        for (int t = 0; t < G::NMK_OWN; ++t) {
          const u32x4 kA =
              lds_tr8<G::WCK>(kb, 16 * ks + 8 * (g4 >> 1), 32 * (mk0 + t) + 16 * (g4 & 1), l16);
          accS[t] = mfma32(kA, vB, accS[t]);
          if constexpr (NORM) {
            // z += sum_t w_t phi(k_t) over this lane's 8 tokens of key 32 (mk0 + t) + l32,
            // two tokens per dot product
            if (stripe == 0) {
#pragma unroll
              for (int e = 0; e < 4; ++e) zacc[t] = dot2_bf16(kA[e], wp[e], zacc[t]);
            }
          }
        }
      }
      if constexpr (CHN && !XF) scale_rows(sEL);
      if constexpr (NORM) {
        if (stripe == 0) {
          const float eLz = (CAT != kCatNone && !STATE_ONLY) ? __builtin_amdgcn_exp2f(bL) : 1.0f;
#pragma unroll
          for (int t = 0; t < G::NMK_OWN; ++t) {
            const float zsum = zacc[t] + __shfl_xor(zacc[t], 32);
            zr[t] = eLz * zr[t] + zsum;
            if (h == 0) sZ[(it + 1) & 1][32 * (mk0 + t) + l32] = zr[t];
          }
        }
      }
    };

    if constexpr (!STATE_ONLY) {
      // (1a) causal score blocks of this wave -> P~ in LDS
#pragma unroll
      for (int bb = 0; bb < G::BPW; ++bb) {
        const int b = wave + NW * bb;
        // (the per-channel decay's exact path has written P~ already)
        if (b < G::NB && !XF) {
          const int I = block_i(b), J = block_j(b);
          f32x16 pacc;
#pragma unroll
          for (int r = 0; r < 16; ++r) pacc[r] = 0.0f;
          // (per-channel decay: the lane's row and half re-derived each chunk, so
          // the compiler forms these swizzled offsets here instead of holding
          // them across the chunk loop, where that kernel's registers run out
          // and they would be spilled -- a scratch reload's wait would also
          // wait for the next chunk's tile copies)
          int ln = lane;
          if constexpr (CHN) asm volatile("" : "+v"(ln));
          const int rl = ln & 31, rh = ln >> 5;
#pragma unroll
          for (int s = 0; s < G::NKS; ++s) {
            const u32x4 kA = lds_b128(kb, swz<G::WCK>(32 * J + rl, 16 * s + 8 * rh));
            const u32x4 qB = lds_b128(qb, swz<G::WCK>(32 * I + rl, 16 * s + 8 * rh));
            pacc = mfma32(kA, qB, pacc);
          }
          // register r: token j = 32 J + 8 (r / 4) + 4 h + r % 4, row i = 32 I + l32
          if constexpr (CHN) {
            // the decay is inside q~ and k~: causal mask only
#pragma unroll
            for (int r = 0; r < 16; ++r)
              pacc[r] = (I != J || 8 * (r >> 2) + 4 * h + (r & 3) <= l32) ? pacc[r] : 0.0f;
          } else if constexpr (CAT == kCatToken) {
            const float bi = sb[32 * I + l32];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 bj = *reinterpret_cast<const f32x4*>(&sb[32 * J + 8 * q + 4 * h]);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float x = pacc[4 * q + e] * __builtin_amdgcn_exp2f(bi - bj[e]);
                pacc[4 * q + e] = (I != J || 8 * q + 4 * h + e <= l32) ? x : 0.0f;
              }
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) pacc[r] *= dm[bb][r];
          }
          const int i = 32 * I + l32;
          if constexpr (NORM) {
            // row i's sum over the block's 32 tokens (16 per lane half)
            float rs = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) rs += pacc[r];
            rs += __shfl_xor(rs, 32);
            if (h == 0) sRS[J][i] = rs;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            u32x2 w;
            w[0] = cvt2(pacc[4 * q + 0], pacc[4 * q + 1]);
            w[1] = cvt2(pacc[4 * q + 2], pacc[4 * q + 3]);
            *reinterpret_cast<u32x2*>(sP + swz<G::WCP>(i, 32 * J + 8 * q + 4 * h)) = w;
          }
        }
      }

      // (1b) inter-chunk term over this wave's keys, every row block:
      //      part[I] = S_part^T Q_part^T (transposed: lane = row, registers = values)
      // (per-channel decay: of diag(e^r) S against q~; the scaled state then
      // carries on into the update)
      // (exact path: the unscaled state against q^ = phi(q) e^{b})
      if constexpr (CHN && !XF) scale_rows(sER);
      pack_state();
      // normalised form: row i's phi(q_i).z over this wave's keys, from the
      // same q pairs as the inter term's operand (lane (i, h) holds 8 of each
      // 16-key step's keys) against z rounded to bf16 pairs, two keys per
      // v_dot2_f32_bf16, the two lane halves then summed.  Row block I's goes
      // to stripe dz_stripe(I), so that stripe 0, which carries the z sums of
      // the state update, takes none of it.
      const float* zc = sZ[it & 1];
      f32x16 pin[G::NRB];
#pragma unroll
      for (int I = 0; I < G::NRB; ++I) {
#pragma unroll
        for (int r = 0; r < 16; ++r) pin[I][r] = 0.0f;
        float dz = 0.0f;
        const int i = 32 * I + l32;
#pragma unroll
        for (int s = 0; s < G::NKS_OWN; ++s) {
          const int sg = part * G::NKS_OWN + s;
          const u32x2 lo = lds_b64(qb, swz<G::WCK>(i, 16 * sg + 4 * h));
          const u32x2 hi = lds_b64(qb, swz<G::WCK>(i, 16 * sg + 8 + 4 * h));
          const u32x4 qop = u32x4{lo[0], lo[1], hi[0], hi[1]};
          pin[I] = mfma32(sbf[s], qop, pin[I]);
          if constexpr (NORM) {
            if (stripe == dz_stripe(I)) {
              const f32x4 z0 = *reinterpret_cast<const f32x4*>(&zc[16 * sg + 4 * h]);
              const f32x4 z1 = *reinterpret_cast<const f32x4*>(&zc[16 * sg + 8 + 4 * h]);
              dz = dot2_bf16(qop[0], cvt2(z0[0], z0[1]), dz);
              dz = dot2_bf16(qop[1], cvt2(z0[2], z0[3]), dz);
              dz = dot2_bf16(qop[2], cvt2(z1[0], z1[1]), dz);
              dz = dot2_bf16(qop[3], cvt2(z1[2], z1[3]), dz);
            }
          }
        }
        if constexpr (NORM) {
          if (stripe == dz_stripe(I)) {
            dz += __shfl_xor(dz, 32);
            if (h == 0) sDen[part][i] = dz;
          }
        }
      }
      // row block I belongs to key part I % KH; the other parts hand it their partial
      if constexpr (KH > 1) {
#pragma unroll
        for (int I = 0; I < G::NRB; ++I)
          if (I % KH != part) {
            char* xb = sX + (size_t)(stripe * G::NRB + I) * 4096 + 16 * lane;
#pragma unroll
            for (int k = 0; k < 4; ++k)
              *reinterpret_cast<f32x4*>(xb + 1024 * k) =
                  f32x4{pin[I][4 * k], pin[I][4 * k + 1], pin[I][4 * k + 2], pin[I][4 * k + 3]};
          }
      }
      lds_barrier();  // P~ and the partials complete

      // (2) outputs of this wave's row blocks: O^T = diag(e^b) (S^T Q^T) + V^T P~^T
#pragma unroll
      for (int I = 0; I < G::NRB; ++I) {
        if (I % KH != part) continue;
        f32x16 acc = pin[I];
        if constexpr (KH > 1) {
          const char* xb = sX + (size_t)(stripe * G::NRB + I) * 4096 + 16 * lane;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(xb + 1024 * k);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[4 * k + e] += x[e];
          }
        }
        const int i = 32 * I + l32;
        float er = 1.0f;
        if constexpr (CAT != kCatNone && !CHN) {
          er = eq[i];
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] *= er;
        }
#pragma unroll
        for (int J = 0; J <= I; ++J)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int ks = 2 * J + s2;
            const u32x4 pB = lds_b128(sP, swz<G::WCP>(i, 16 * ks + 8 * h));
            acc = mfma32(vA[ks], pB, acc);
          }
        if constexpr (NORM) {
          // denominator of row i: e^{b_i} phi(q_i).z_c + its masked score row sum
          float dz = 0.0f, ds = 0.0f;
#pragma unroll
          for (int p = 0; p < KH; ++p) dz += sDen[p][i];
#pragma unroll
          for (int J = 0; J <= I; ++J) ds += sRS[J][i];
          const float inv = 1.0f / (er * dz + ds);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] *= inv;
        }
        // lane: row i, value columns cw + 8 q + 4 h + (0..3) -> LDS slot,
        // then 16-byte pieces of whole rows -> HBM
        char* so = sO[wave];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u32x2 w;
          w[0] = cvt2(acc[4 * q + 0], acc[4 * q + 1]);
          w[1] = cvt2(acc[4 * q + 2], acc[4 * q + 3]);
          *reinterpret_cast<u32x2*>(so + swz<4>(l32, 8 * q + 4 * h)) = w;
        }
        lds_wave_sync();
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int row = (lane >> 2) + 16 * it, cc = lane & 3;
          const u32x4 w = lds_b128(so, swz<4>(row, 8 * cc));
          if (32 * I + row < nvalid)
            __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(oh + (size_t)(t0 + 32 * I + row) * DV + 8 * cc));
        }
        lds_wave_sync();
      }
    }

    state_update();
    logA += bL;
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  if (n_it > 0) issue_loads(S0{}, 0);
  if constexpr (NS == 3) {
    if (n_it > 1) issue_loads(S1{}, 1);
    for (int it = 0; it < n_it; it += 3) {
      body(S0{}, it);
      if (it + 1 < n_it) body(S1{}, it + 1);
      if (it + 2 < n_it) body(S2{}, it + 2);
    }
  } else {
    for (int it = 0; it < n_it; it += 2) {
      body(S0{}, it);
      if (it + 1 < n_it) body(S1{}, it + 1);
    }
  }

  // ---- epilogue ---------------------------------------------------------
  // (every thread's flag write came before a barrier of the last chunk)
  if constexpr (CHN && !STATE_ONLY && !EXACT)
    if (tid == 0) a.ws_flag[f] = sBad;
  if constexpr (STATE_ONLY) {
    if (copy_s0) {
#pragma unroll
      for (int t = 0; t < G::NMK_OWN; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) a.ws_S0[s0_index(t, r)] = s0v[t][r];
    }
  }
  float* dst = nullptr;
  if constexpr (STATE_ONLY) {
    dst = a.ws_S + (unit0 + sigma) * DK * DV;
    if constexpr (CHN) {
      if (vt == 0 && run == 0)
        *reinterpret_cast<fcv*>(&a.ws_logA[(unit0 + sigma) * DK + ch0]) = logAc;
    } else {
      if (vt == 0 && tid == 0) a.ws_logA[unit0 + sigma] = logA;
    }
  } else {
    if (sigma == a.P - 1 && a.state != nullptr) dst = a.state + (size_t)bh * DK * DV;
  }
  if (dst != nullptr) {
    const int dv = dv0 + cw + l32;
#pragma unroll
    for (int t = 0; t < G::NMK_OWN; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        dst[(size_t)(32 * (mk0 + t) + 8 * (r >> 2) + 4 * h + (r & 3)) * DV + dv] = accS[t][r];
  }
  if constexpr (NORM) {
    float* zdst = nullptr;
    if constexpr (STATE_ONLY) zdst = a.ws_z + (unit0 + sigma) * DK;
    else if (sigma == a.P - 1 && a.zstate != nullptr) zdst = a.zstate + (size_t)bh * DK;
    if (zdst != nullptr && stripe == 0 && h == 0 && vt == 0) {
#pragma unroll
      for (int t = 0; t < G::NMK_OWN; ++t) zdst[32 * (mk0 + t) + l32] = zr[t];
    }
  }
}

// ---- launch and dispatch ----------------------------------------------------
template <int DK, int NWV, int KH, int C, int CAT>
hipError_t launch_one(const ChunkArgs& a, bool state_only, hipStream_t s) {
  const int groups = (a.n_units + 7) / 8;
  const dim3 grid(groups * 8 * a.n_v), block(64 * NWV * KH);
  if constexpr (CAT == kCatChannel) {
    if (a.norm || (!state_only && a.ws_flag == nullptr)) return hipErrorInvalidValue;
    if (state_only) {
      hipLaunchKernelGGL((chunk_stripe_kernel<DK, NWV, KH, C, CAT, true, false>), grid, block, 0, s, a);
    } else {
      // the split pass flags the workgroups that met a chunk too strongly
      // decayed for it; the exact pass recomputes those and exits elsewhere
      hipLaunchKernelGGL((chunk_stripe_kernel<DK, NWV, KH, C, CAT, false, false>), grid, block, 0, s, a);
      hipLaunchKernelGGL((chunk_stripe_kernel<DK, NWV, KH, C, CAT, false, false, true>), grid, block, 0, s, a);
    }
  } else if (a.norm) {
    if (state_only)
      hipLaunchKernelGGL((chunk_stripe_kernel<DK, NWV, KH, C, CAT, true, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((chunk_stripe_kernel<DK, NWV, KH, C, CAT, false, true>), grid, block, 0, s, a);
  } else {
    if (state_only)
      hipLaunchKernelGGL((chunk_stripe_kernel<DK, NWV, KH, C, CAT, true, false>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((chunk_stripe_kernel<DK, NWV, KH, C, CAT, false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <int DK, int NWV, int KH, int C, int CAT>
constexpr bool fits() {
  using G = Geo<DK, NWV, KH, C, false, CAT == kCatChannel>;
  return G::LDS <= kMaxLds && G::CH_OK;
}

template <int DK, int NWV, int KH, int CAT>
hipError_t dispatch_c(const ChunkArgs& a, bool so, hipStream_t s) {
  switch (a.C) {
    case 32:
      if constexpr (fits<DK, NWV, KH, 32, CAT>()) return launch_one<DK, NWV, KH, 32, CAT>(a, so, s);
      return hipErrorInvalidValue;
    case 64:
      if constexpr (fits<DK, NWV, KH, 64, CAT>()) return launch_one<DK, NWV, KH, 64, CAT>(a, so, s);
      return hipErrorInvalidValue;
    case 128:
      if constexpr (fits<DK, NWV, KH, 128, CAT>()) return launch_one<DK, NWV, KH, 128, CAT>(a, so, s);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

// a.tv is the workgroup's value width (32, 64 or 128 columns: 1, 2, 4
// stripes); a.ng the number of key parts per stripe (1 or 2)
template <int DK, int CAT>
hipError_t dispatch_w(const ChunkArgs& a, bool so, hipStream_t s) {
  if (a.ng == 2) {
    if constexpr (DK >= 64) {
      switch (a.tv) {
        case 32: return dispatch_c<DK, 1, 2, CAT>(a, so, s);
        case 64: return dispatch_c<DK, 2, 2, CAT>(a, so, s);
        case 128: return dispatch_c<DK, 4, 2, CAT>(a, so, s);
      }
    }
    return hipErrorInvalidValue;
  }
  switch (a.tv) {
    case 32: return dispatch_c<DK, 1, 1, CAT>(a, so, s);
    case 64: return dispatch_c<DK, 2, 1, CAT>(a, so, s);
    case 128: return dispatch_c<DK, 4, 1, CAT>(a, so, s);
  }
  return hipErrorInvalidValue;
}

template <int DK, int NWV, int KH>
constexpr bool fits_c(int C, bool ch) {
  if (ch)
    return C == 32 ? fits<DK, NWV, KH, 32, kCatChannel>()
                   : C == 64 ? fits<DK, NWV, KH, 64, kCatChannel>() : fits<DK, NWV, KH, 128, kCatChannel>();
  return C == 32 ? fits<DK, NWV, KH, 32, kCatToken>()
                 : C == 64 ? fits<DK, NWV, KH, 64, kCatToken>() : fits<DK, NWV, KH, 128, kCatToken>();
}
// Whether the layout (TVW value columns, KH key parts, chunk C) fits: the
// per-token category stands for the three factorised ones (they share one
// LDS plan), the per-channel one has its own.
template <int DK>
constexpr bool fits_of(int TVW, int KH, int C, bool ch) {
  if constexpr (DK >= 64) {
    if (KH == 2)
      return TVW == 32 ? fits_c<DK, 1, 2>(C, ch) : TVW == 64 ? fits_c<DK, 2, 2>(C, ch) : fits_c<DK, 4, 2>(C, ch);
  }
  return TVW == 32 ? fits_c<DK, 1, 1>(C, ch) : TVW == 64 ? fits_c<DK, 2, 1>(C, ch) : fits_c<DK, 4, 1>(C, ch);
}

}  // namespace stripe

// One per (key dimension, decay category), each in its own translation unit.
#define LA_STRIPE_DECL(DK, CAT) \
  hipError_t launch_chunk_stripe_dk##DK##_c##CAT(const ChunkArgs& a, bool state_only, hipStream_t s);
LA_STRIPE_DECL(32, 0) LA_STRIPE_DECL(32, 1) LA_STRIPE_DECL(32, 2) LA_STRIPE_DECL(32, 3)
LA_STRIPE_DECL(64, 0) LA_STRIPE_DECL(64, 1) LA_STRIPE_DECL(64, 2) LA_STRIPE_DECL(64, 3)
LA_STRIPE_DECL(128, 0) LA_STRIPE_DECL(128, 1) LA_STRIPE_DECL(128, 2) LA_STRIPE_DECL(128, 3)
#undef LA_STRIPE_DECL

}  // namespace la
