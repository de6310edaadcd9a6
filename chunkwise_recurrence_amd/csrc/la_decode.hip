// la_decode.hip -- the recurrent one-token step and the state fill.
//
// Per head (linear_attn_recurrent of "Linear / Sparse Attention - minimal
// runnable implementation", one iteration; decay as in CS336 lecture 4 code 1,
// gated_linear_attention_recurrent):
//
//   S' = a S + phi(k) v^T,   o = phi(q)^T S'
//
// The normalised form also updates z' = a z + phi(k) and divides o by
// phi(q)^T z' (the tutorial's section 2.2, boxed recurrence).  With the
// per-channel gate (the tutorial's section 2.4) a is a vector over the key
// channels: row i of S and entry i of z decay by a_i.
//
// The delta rule (DeltaNet, gated by a scalar a; "Linear / Sparse Attention",
// delta_rule_recurrent, stored transposed) first reads what the old state
// returns for k, r = k^T S, then writes S' = a (S - beta k r^T) + beta k v^T:
// one more reduction over the rows the lanes already hold.
//
// The step is a pure stream over the fp32 state: every element is read once,
// updated and written once, and o is reduced on the way.  One workgroup of 256
// lanes per head; each lane owns 4 adjacent columns (one 16-byte vector) of
// DK / (256 / (DV/4)) rows, so a row of the state is read by DV/4 consecutive
// lanes in one coalesced 16-byte-per-lane access.  All of a lane's state loads
// are issued before any arithmetic, then the partial sums of o over a lane's
// rows are combined across row groups through LDS.  The state is touched once
// per step and is larger than every cache, so its loads and stores carry the
// non-temporal hint.
#include "la_device.h"

namespace la {
namespace {

// VAR: 0 a scalar decay (or none), 1 the per-channel decay, 2 the delta rule
template <int DK, int DV, bool BF16, int VAR>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeArgs a) {
  constexpr bool DELTA = VAR == 2, CHAN = VAR == 1;
  constexpr int TPR = DV / 4;                      // lanes per state row
  constexpr int RP = 256 / TPR;                    // rows per pass
  constexpr int NPASS = (DK + RP - 1) / RP;
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int h = bh % a.H;
  const int rg = tid / TPR, c4 = tid % TPR;

  typedef float f32x4 __attribute__((ext_vector_type(4)));
  f32x4* S = reinterpret_cast<f32x4*>(a.state + (size_t)bh * DK * DV);
  f32x4 sreg[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int r = rg + p * RP;
    if (r < DK) sreg[p] = __builtin_nontemporal_load(&S[r * TPR + c4]);
  }

  __shared__ float sq[DK], sk[DK], sv[DV];
  __shared__ float red[RP][DV + 4];
  const bool elu = a.phi == kPhiElu1;
  if (tid < DK) {
    float qv, kv;
    if constexpr (BF16) {
      qv = bf16_to_f32(static_cast<const uint16_t*>(a.q)[(size_t)bh * DK + tid]);
      kv = bf16_to_f32(static_cast<const uint16_t*>(a.k)[(size_t)bh * DK + tid]);
    } else {
      qv = static_cast<const float*>(a.q)[(size_t)bh * DK + tid];
      kv = static_cast<const float*>(a.k)[(size_t)bh * DK + tid];
    }
    sq[tid] = elu ? feature_elu1_accurate(qv) : qv;
    sk[tid] = elu ? feature_elu1_accurate(kv) : kv;
  }
  if (tid < DV) {
    if constexpr (BF16) sv[tid] = bf16_to_f32(static_cast<const uint16_t*>(a.v)[(size_t)bh * DV + tid]);
    else sv[tid] = static_cast<const float*>(a.v)[(size_t)bh * DV + tid];
  }
  float decay = 1.0f;
  if (a.decay_kind == kDecayHead) decay = a.decay[h];
  else if (a.decay_kind == kDecayLog || a.decay_kind == kDecayGate)
    decay = expf(token_log_decay(a.decay_kind, a.decay[bh]));
  __shared__ float sdec[DK];
  if (tid < DK) sdec[tid] = CHAN ? expf(a.decay[(size_t)bh * DK + tid]) : decay;
  // delta rule: r = k^T S of the previous state, reduced over the row groups
  __shared__ float sr[DELTA ? DV : 1];
  float bta = 0.0f;
  if constexpr (DELTA) {
    bta = a.beta[bh];
    __syncthreads();
    float4 rp = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int r = rg + p * RP;
      if (r < DK) {
        const float kr = sk[r];
        rp.x = fmaf(kr, sreg[p].x, rp.x);
        rp.y = fmaf(kr, sreg[p].y, rp.y);
        rp.z = fmaf(kr, sreg[p].z, rp.z);
        rp.w = fmaf(kr, sreg[p].w, rp.w);
      }
    }
    if (rg < RP) {
      red[rg][4 * c4] = rp.x;
      red[rg][4 * c4 + 1] = rp.y;
      red[rg][4 * c4 + 2] = rp.z;
      red[rg][4 * c4 + 3] = rp.w;
    }
    __syncthreads();
    if (tid < DV) {
      float acc = 0.0f;
      constexpr int used = DK < RP ? DK : RP;
#pragma unroll
      for (int g = 0; g < used; ++g) acc += red[g][tid];
      sr[tid] = acc;
    }
  }
  __shared__ float sden[DK];
  if (a.zstate != nullptr) {
    __syncthreads();
    if (tid < DK) {
      float* zp = a.zstate + (size_t)bh * DK + tid;
      const float z = fmaf(sdec[tid], *zp, sk[tid]);
      *zp = z;
      sden[tid] = sq[tid] * z;
    }
  }
  __syncthreads();

  const float4 vv = make_float4(sv[4 * c4], sv[4 * c4 + 1], sv[4 * c4 + 2], sv[4 * c4 + 3]);
  float4 rv = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (DELTA) rv = make_float4(sr[4 * c4], sr[4 * c4 + 1], sr[4 * c4 + 2], sr[4 * c4 + 3]);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int r = rg + p * RP;
    if (r < DK) {
      const float kr = sk[r], qr = sq[r];
      const float dr = CHAN ? sdec[r] : decay;
      f32x4 s = sreg[p];
      if constexpr (DELTA) {
        // S' = a (S - beta k r^T) + beta k v^T
        const float bk = bta * kr;
        s.x = fmaf(dr, fmaf(-bk, rv.x, s.x), bk * vv.x);
        s.y = fmaf(dr, fmaf(-bk, rv.y, s.y), bk * vv.y);
        s.z = fmaf(dr, fmaf(-bk, rv.z, s.z), bk * vv.z);
        s.w = fmaf(dr, fmaf(-bk, rv.w, s.w), bk * vv.w);
      } else {
        s.x = fmaf(dr, s.x, kr * vv.x);
        s.y = fmaf(dr, s.y, kr * vv.y);
        s.z = fmaf(dr, s.z, kr * vv.z);
        s.w = fmaf(dr, s.w, kr * vv.w);
      }
      __builtin_nontemporal_store(s, &S[r * TPR + c4]);
      o.x = fmaf(qr, s.x, o.x);
      o.y = fmaf(qr, s.y, o.y);
      o.z = fmaf(qr, s.z, o.z);
      o.w = fmaf(qr, s.w, o.w);
    }
  }
  if (rg < RP) {
    red[rg][4 * c4] = o.x;
    red[rg][4 * c4 + 1] = o.y;
    red[rg][4 * c4 + 2] = o.z;
    red[rg][4 * c4 + 3] = o.w;
  }
  __syncthreads();
  if (tid < DV) {
    float acc = 0.0f;
    constexpr int used = DK < RP ? DK : RP;
#pragma unroll
    for (int g = 0; g < used; ++g) acc += red[g][tid];
    if (a.zstate != nullptr) {
      float den = 0.0f;
      for (int d = 0; d < DK; ++d) den += sden[d];
      acc /= den;
    }
    if constexpr (BF16)
      static_cast<uint16_t*>(a.out)[(size_t)bh * DV + tid] = (uint16_t)f32_to_bf16(acc);
    else
      static_cast<float*>(a.out)[(size_t)bh * DV + tid] = acc;
  }
}

template <int DK, int DV>
hipError_t launch_dk_dv(const DecodeArgs& a, int dtype, hipStream_t s) {
  const dim3 grid(a.N * a.H), block(256);
  const int var = a.beta != nullptr ? 2 : a.decay_kind == kDecayChannel ? 1 : 0;
#define LA_VAR(V)                                                                           \
  if (var == V) {                                                                           \
    if (dtype == kBF16) hipLaunchKernelGGL((decode_kernel<DK, DV, true, V>), grid, block, 0, s, a); \
    else hipLaunchKernelGGL((decode_kernel<DK, DV, false, V>), grid, block, 0, s, a);      \
    return hipGetLastError();                                                               \
  }
  LA_VAR(0)
  LA_VAR(1)
  LA_VAR(2)
#undef LA_VAR
  return hipErrorInvalidValue;
}

template <int DK>
hipError_t launch_dv(const DecodeArgs& a, int dtype, hipStream_t s) {
  switch (a.DV) {
    case 16: return launch_dk_dv<DK, 16>(a, dtype, s);
    case 32: return launch_dk_dv<DK, 32>(a, dtype, s);
    case 64: return launch_dk_dv<DK, 64>(a, dtype, s);
    case 128: return launch_dk_dv<DK, 128>(a, dtype, s);
  }
  return hipErrorInvalidValue;
}

__global__ void fill_zero_kernel(float4* p, size_t n4) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// dst[i] = src[i] for n floats in 16-byte pieces (n a multiple of 4, both
// 16-byte aligned).
__global__ void copy_f32_kernel(float4* dst, const float4* src, size_t n4) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t s) {
  switch (a.DK) {
    case 16: return launch_dv<16>(a, dtype, s);
    case 32: return launch_dv<32>(a, dtype, s);
    case 64: return launch_dv<64>(a, dtype, s);
    case 128: return launch_dv<128>(a, dtype, s);
  }
  return hipErrorInvalidValue;
}

// n is a multiple of 4 (d_v is a multiple of 16 and the pointer 16-byte aligned).
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s) {
  const size_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<float4*>(p), n4);
  return hipGetLastError();
}

hipError_t launch_copy_f32(float* dst, const float* src, size_t n, hipStream_t s) {
  const size_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(copy_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<float4*>(dst), reinterpret_cast<const float4*>(src), n4);
  return hipGetLastError();
}

}  // namespace la
