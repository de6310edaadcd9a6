// la_internal.h -- launch descriptors shared by the host API (la_api.hip) and
// the kernel files.  Not part of the public ABI (that is include/la.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace la {

// Public enum values, mirrored for device code.
enum { kF32 = 0, kBF16 = 1 };
enum { kPhiIdentity = 0, kPhiElu1 = 1 };
enum { kDecayNone = 0, kDecayHead = 1, kDecayLog = 2, kDecayGate = 3, kDecayChannel = 4 };

// One la_chunk_fwd launch (main pass or segment-state pass).
struct ChunkArgs {
  const void* q;        // [B,H,L,DK]
  const void* k;        // [B,H,L,DK]
  const void* v;        // [B,H,L,DV]
  void* out;            // [B,H,L,DV]
  float* state;         // [B,H,DK,DV] or nullptr; S_0 in, S_L out
  // Where the output pass reads S_0 and z_0.  A head whose work spans several
  // workgroups must not read them from state / zstate, which the workgroup of
  // its last segment (or first value tile) overwrites with S_L / z_L: then
  // they are copies in the workspace (S_0 copied by the state pass, z_0 by a
  // copy launched before the passes).
  const float* s0;      // [B,H,DK,DV] or nullptr (S_0 = 0)
  const float* z0;      // normalised form: [B,H,DK] or nullptr (z_0 = 0)
  float* ws_S0;         // state pass: where it copies S_0 (nullptr: no copy)
  const float* decay;   // nullptr | gamma[H] | [B,H,L] | [B,H,L,DK] (per channel)
  float* ws_S;          // [B*H, P*sub, DK, DV] state increments of the state-pass units
  float* ws_logA;       // [B*H, P*sub] their total log2 decays ([B*H, P*sub, DK] per channel)
  float* ws_b;          // [B*H, L] in-chunk inclusive prefix of log a (token decays)
  float* zstate;        // normalised form: [B,H,DK] z in/out, or nullptr
  float* ws_z;          // normalised form: [B*H, P*sub, DK] z increments of the state-pass units
  int* ws_flag;         // per-channel decay (stripe kernel): one flag per output-pass
                        // workgroup, set when its segment needs the exact re-run
  int norm;             // 1: the normalised form
  int B, H, L, DK, DV, C;
  int P;                // sequence segments per head
  int seg_chunks;       // chunks per segment (the last one may hold fewer)
  int sub;              // state-pass units per segment (a divisor of seg_chunks; each
                        // covers seg_chunks / sub chunks), composed like segments
  int n_units;          // work units: B*H*P (main) or B*H*(P-1)*sub (state pass)
  int n_v;              // value tiles per head (one workgroup each)
  int tv;               // strip kernel: value columns per column group; stripe kernel: per workgroup
  int ng;               // strip kernel: column groups (of 4 waves) per workgroup;
                        // stripe kernel: key parts per 32-column stripe
  int phi, decay_kind;
};

// Largest chunk the delta-rule kernels take.
constexpr int kDeltaMaxC = 64;

// One la_delta_fwd: the chunk-parallel solve pass and the sequential pass.
struct DeltaArgs {
  const void* q;        // [B,H,L,DK]
  const void* k;        // [B,H,L,DK]
  const void* v;        // [B,H,L,DV]
  const float* beta;    // [B,H,L]
  void* out;            // [B,H,L,DV]
  float* state;         // [B,H,DK,DV] or nullptr
  const float* decay;   // nullptr | gamma[H] | [B,H,L]
  float* ws_W;          // [B*H, L, DK] W = T diag(beta e^b) K per chunk
  float* ws_U;          // [B*H, L, DV] U0 = T diag(beta) V per chunk (bf16 on the
                        // matrix-core path, in the first half of the region)
  void* ws_P;           // matrix-core path: [B*H, L, kDeltaMaxC] bf16 rows of each chunk's
                        // causal scores (q_i . k_j) e^{b_i - b_j} [j <= i]
  float* ws_b;          // matrix-core path: [B*H, L] in-chunk inclusive prefix of log2 a,
                        // written by the solve pass for the sequential pass
  int B, H, L, DK, DV, C;
  int decay_kind, dtype;
  int n_v;              // value tiles per head
};

// The delta rule's matrix-core path (bf16 inputs, 64-token chunks, d_k >= 32,
// whole 32-column value tiles); other problems take the fp32-arithmetic
// kernels.
inline bool delta_uses_mfma(int dtype, int C, int DK, int DV) {
  return dtype == kBF16 && C == 64 && DK >= 32 && DV % 32 == 0;
}

struct DecodeArgs {
  const void* q;        // [N,H,DK]
  const void* k;        // [N,H,DK]
  const void* v;        // [N,H,DV]
  void* out;            // [N,H,DV]
  float* state;         // [N,H,DK,DV]
  float* zstate;        // normalised form: [N,H,DK], or nullptr
  const float* beta;    // delta rule: [N,H] write strengths, or nullptr
  const float* decay;   // nullptr | gamma[H] | [N,H] | [N,H,DK] (per channel)
  int N, H, DK, DV;
  int phi, decay_kind;
};

// Launchers (return the launch error, hipSuccess when enqueued).
hipError_t launch_chunk_bf16(const ChunkArgs& a, bool state_only, hipStream_t s);
hipError_t launch_chunk_stripe(const ChunkArgs& a, bool state_only, hipStream_t s);
hipError_t launch_decay_prefix(const ChunkArgs& a, hipStream_t s);
hipError_t launch_chunk_f32(const ChunkArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t s);
hipError_t launch_delta(const DeltaArgs& a, hipStream_t s);
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s);
hipError_t launch_copy_f32(float* dst, const float* src, size_t n, hipStream_t s);

// Whether a bf16 kernel exists for key dim DK, NG column groups of TV columns
// and chunk C (and fits the LDS).
bool chunk_bf16_supported(int DK, int TV, int NG, int C);
// Whether the stripe kernel exists for key dim DK, TVW value columns per
// workgroup, KH key parts per stripe and chunk C (and fits the LDS).
// With `channel`, for the per-channel decay.
bool chunk_stripe_supported(int DK, int TVW, int KH, int C, bool channel = false);

}  // namespace la
