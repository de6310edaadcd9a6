// la_api.hip -- the C ABI of liblinattn.so (declared in include/la.h):
// argument validation on the host, the launch plan, and the launches.
//
// Validation happens before any launch, so every error path can be exercised
// on a machine without a GPU (the plan asks the runtime for the current
// device's compute units, and assumes an MI355X's 256 when none is visible).
#include <atomic>
#include <mutex>
#include <stdint.h>

#include "la.h"
#include "la_internal.h"

namespace {

// A segment of the sequence keeps at least this many chunks.
constexpr int kMinSegmentChunks = 4;
// Compute units assumed when no device is visible (plan queries on a host
// without a GPU): an MI355X.
constexpr int kDefaultComputeUnits = 256;
constexpr int kMaxDevices = 64;

// The library's only global state: compute units per device, queried once
// per device and cached (0 = not yet known).  Concurrent first calls may both
// query; they store the same value.
std::atomic<int> g_device_cus[kMaxDevices];

int device_compute_units() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kDefaultComputeUnits;
  }
  int n = g_device_cus[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n < 1) {
    (void)hipGetLastError();
    return kDefaultComputeUnits;
  }
  g_device_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Scratch for la_chunk_fwd_noalloc: a fixed device array instead of a caller
// workspace.  Each device the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: host code uses only the address hipGetSymbolAddress returns
// for the current device (g_scratch_ptr).
constexpr size_t kScratchBytes = LA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The current device's scratch address, looked up once per device with that
// device current.  nullptr if the lookup failed.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    if (g_scratch_err[dev] != hipSuccess) (void)hipGetLastError();
  });
  return g_scratch_ptr[dev];
}

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

struct Plan {
  int kernel = 0;    // LA_KERNEL_F32, LA_KERNEL_STRIP or LA_KERNEL_STRIPE
  int tile = 0;      // value columns of one workgroup
  int ng = 1;        // column groups (of 4 waves) per workgroup (bf16 path)
  int tv = 0;        // value columns per column group
  int P = 1;         // sequence segments per head
  int seg_chunks = 0;
  int sub = 1;       // state-pass units per segment (a divisor of seg_chunks)
  size_t ws_bytes = 0;
  size_t ws_S_off = 0, ws_logA_off = 0, ws_b_off = 0, ws_z_off = 0;
  // copies of S_0 (segment split) and z_0 (normalised form, a head spread over
  // several workgroups); 0 = none
  size_t ws_S0_off = 0, ws_z0_off = 0;
  bool copy_S0 = false, copy_z0 = false;
  // per-channel decay (stripe kernel): one flag per output-pass workgroup for
  // the exact re-run, and (one segment) a copy of S_0 that re-run reads, since
  // the first pass has overwritten the caller's state with S_L by then
  size_t ws_flag_off = 0;
  bool flags = false, copy_S0_host = false;
  bool prefix = false;  // token decays: in-chunk prefix sums of log a in the workspace
};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

bool t_fits(int d_k, int tile, int ng, int C) {
  return tile % ng == 0 && la::chunk_bf16_supported(d_k, tile / ng, ng, C);
}

la_status check_chunk_shape(int dtype, int B, int H, int L, int d_k, int d_v, int C) {
  if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || L < 0 || C < 1) return LA_ERR_SHAPE;
  if (!dim_ok(d_k) || !dim_ok(d_v) || !dim_ok(C)) return LA_ERR_UNSUPPORTED;
  return LA_OK;
}

// A caller's plan request: every field 0 = automatic.
la_status check_request(const la_plan* r) {
  if (!r) return LA_OK;
  if (r->kernel != 0 && r->kernel != LA_KERNEL_STRIP && r->kernel != LA_KERNEL_STRIPE)
    return LA_ERR_UNSUPPORTED;
  if (r->dv_tile != 0 && !dim_ok(r->dv_tile)) return LA_ERR_UNSUPPORTED;
  if (r->groups != 0 && r->groups != 1 && r->groups != 2) return LA_ERR_UNSUPPORTED;
  if (r->segments < 0 || r->state_split < 0) return LA_ERR_SHAPE;
  return LA_OK;
}

Plan make_plan(int B, int H, int L, int d_k, int d_v, int C, int dtype, int decay_kind,
               bool norm, const la_plan* request) {
  Plan p;
  const int heads = B * H;
  const int nchunks = L > 0 ? (L + C - 1) / C : 0;
  if (dtype == LA_F32) {
    p.kernel = LA_KERNEL_F32;
    p.tile = p.tv = d_v < 32 ? d_v : 32;
    p.ng = 1;
    p.P = 1;
    p.seg_chunks = nchunks;
    if (norm && d_v / p.tile > 1) {
      p.copy_z0 = true;
      p.ws_z0_off = 0;
      p.ws_bytes = round256((size_t)heads * d_k * sizeof(float));
    }
    return p;
  }
  const la_plan none{};
  const la_plan& req = request ? *request : none;
  const int forced_kernel = req.kernel, forced_tile = req.dv_tile, forced_groups = req.groups;
  // 128-wide heads: the stripe kernel (32x32 MFMA, the state in registers,
  // one 8-wave workgroup per head and segment).  Narrower heads, 16-token
  // chunks and shapes the stripe kernel does not cover: the strip kernel
  // (16x16 MFMA, 4-wave workgroups over 32-column tiles, siblings sharing q
  // and k through L2).  Both measured on MI355X; a caller's plan request
  // (la_chunk_fwd_planned) overrides.
  int tile = 0;
  // the normalised form and the per-channel decay run in the stripe kernel only
  const bool chan = decay_kind == LA_DECAY_CHANNEL_LOG;
  const bool stripe_only = norm || chan;
  const bool stripe_auto = stripe_only || (d_v == 128 && d_k >= 64);
  if (stripe_only || forced_kernel == LA_KERNEL_STRIPE || (forced_kernel == 0 && stripe_auto)) {
    // two waves per 32-column stripe (each holding half of the keys) where
    // d_k allows, for two waves per SIMD
    auto parts_for = [&](int t) {
      if (forced_groups > 0) return forced_groups;
      return la::chunk_stripe_supported(d_k, t, 2, C, chan) ? 2 : 1;
    };
    tile = forced_tile > 0 ? forced_tile : d_v;
    while (tile > d_v) tile /= 2;
    while (tile >= 32 && !la::chunk_stripe_supported(d_k, tile, parts_for(tile), C, chan)) tile /= 2;
    if (tile >= 32) {
      p.kernel = LA_KERNEL_STRIPE;
      p.tile = p.tv = tile;
      p.ng = parts_for(tile);
    }
  }
  if (p.kernel == 0) {
    p.kernel = LA_KERNEL_STRIP;
    // 64-wide value heads with d_k >= 64: one 64-column tile in two groups
    // (the siblings share the q and k tiles in LDS instead of through L2);
    // measured on MI355X: 4-17 % faster over the shapes tried, even at C = 32,
    // 6 % slower at d_k = 32
    const bool wide64 = forced_tile == 0 && d_v == 64 && d_k >= 64;
    tile = forced_tile > 0 ? forced_tile : wide64 ? 64 : (d_v < 32 ? d_v : 32);
    while (tile > d_v) tile /= 2;
    auto groups_for = [&](int t) {
      int g = forced_groups > 0 ? forced_groups : (wide64 && t == 64 ? 2 : 1);
      if (t / g < 16) g = 1;
      return g;
    };
    // the widest layout that has a kernel and fits the LDS
    while (tile > 16 && !(t_fits(d_k, tile, groups_for(tile), C))) tile /= 2;
    p.tile = tile;
    p.ng = groups_for(tile);
    p.tv = tile / p.ng;
  }
  int P = 1;
  // count the strip kernel's 4-wave column groups, so that a two-group tile
  // gets the segment count of two one-group tiles
  const long long units =
      (long long)heads * (d_v / tile) * (p.kernel == LA_KERNEL_STRIP ? p.ng : 1);
  // one 8-wave stripe workgroup per compute unit, or two 4-wave strip
  // workgroups per compute unit
  const int cus = device_compute_units();
  const long long target = p.kernel == LA_KERNEL_STRIPE ? cus : 2LL * cus;
  while (units * P < target && (long long)P * 2 * kMinSegmentChunks <= nchunks) P *= 2;
  const int forced_P = req.segments;
  if (forced_P > 0) P = forced_P;
  if (P > nchunks) P = nchunks;
  if (P < 1) P = 1;
  p.seg_chunks = nchunks > 0 ? (nchunks + P - 1) / P : 0;
  p.P = p.seg_chunks > 0 ? (nchunks + p.seg_chunks - 1) / p.seg_chunks : 1;
  if (p.P > 1) {
    // The strip kernel's state pass (light workgroups, three per compute unit
    // fit) is split until its grid covers the compute units, at most in four:
    // elu_bf16's 192 state workgroups become 384, 17.0 -> 13.6 us on MI355X,
    // the output pass unchanged (it composes twice as many increments; four
    // splits cost it 2 us).  The stripe kernel's state pass measured no
    // faster split (retnet_bf16 reads at the HBM rate already).
    int sub = 1;
    if (p.kernel == LA_KERNEL_STRIP) {
      const long long state_wgs = (long long)heads * (d_v / p.tile) * (p.P - 1);
      while (sub < 4 && state_wgs * sub < cus && p.seg_chunks % (2 * sub) == 0) sub *= 2;
    }
    if (req.state_split > 0) sub = req.state_split;
    if (sub > p.seg_chunks) sub = p.seg_chunks;
    while (p.seg_chunks % sub != 0) --sub;
    p.sub = sub;
  }
  size_t off = 0;
  if (p.P > 1) {
    // one slot per state-pass unit: P * sub per head (the last segment's unused)
    const size_t units = (size_t)heads * p.P * p.sub;
    p.ws_S_off = off;
    off += round256(units * d_k * d_v * sizeof(float));
    p.ws_logA_off = off;  // one total per unit, or per unit and key channel
    off += round256(units * (chan ? d_k : 1) * sizeof(float));
    p.ws_z_off = off;  // the normalised form's z increments
    off += round256(units * d_k * sizeof(float));
    p.copy_S0 = true;
    p.ws_S0_off = off;
    off += round256((size_t)heads * d_k * d_v * sizeof(float));
  }
  if (chan && p.kernel == LA_KERNEL_STRIPE) {
    const long long groups = ((long long)heads * p.P + 7) / 8;
    p.flags = true;
    p.ws_flag_off = off;
    off += round256((size_t)groups * 8 * (d_v / p.tile) * sizeof(int));
    if (p.P == 1) {
      p.copy_S0_host = true;
      p.ws_S0_off = off;
      off += round256((size_t)heads * d_k * d_v * sizeof(float));
    }
  }
  if (norm && (p.P > 1 || d_v / p.tile > 1)) {
    p.copy_z0 = true;
    p.ws_z0_off = off;
    off += round256((size_t)heads * d_k * sizeof(float));
  }
  if (decay_kind == LA_DECAY_TOKEN_LOG || decay_kind == LA_DECAY_TOKEN_GATE) {
    p.prefix = true;
    p.ws_b_off = off;
    off += round256((size_t)heads * L * sizeof(float));
  }
  p.ws_bytes = off;
  return p;
}

}  // namespace

extern "C" {

const char* la_status_string(int s) {
  switch (s) {
    case LA_OK: return "LA_OK";
    case LA_ERR_NULL: return "LA_ERR_NULL: a required pointer is NULL";
    case LA_ERR_SHAPE: return "LA_ERR_SHAPE: B, H or N < 1, L < 0 or C < 1";
    case LA_ERR_UNSUPPORTED:
      return "LA_ERR_UNSUPPORTED: d_k, d_v or C not in {16,32,64,128}, or an unknown dtype/phi/decay";
    case LA_ERR_ALIGN: return "LA_ERR_ALIGN: a pointer is not 16-byte aligned";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE: workspace missing or too small";
    case LA_ERR_DEVICE: return "LA_ERR_DEVICE: a HIP call or kernel launch failed";
  }
  return "unknown la_status";
}

la_status la_chunk_fwd_plan(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                            int decay_kind, int normalize, la_plan* plan,
                            size_t* workspace_bytes) {
  const la_status st = check_chunk_shape(dtype, B, H, L, d_k, d_v, C);
  if (st != LA_OK) return st;
  if (decay_kind < LA_DECAY_NONE || decay_kind > LA_DECAY_CHANNEL_LOG) return LA_ERR_UNSUPPORTED;
  if (!plan) return LA_ERR_NULL;
  const la_status rs = check_request(plan);
  if (rs != LA_OK) return rs;
  const la_plan request = *plan;
  const Plan p = make_plan(B, H, L, d_k, d_v, C, dtype, decay_kind, normalize != 0, &request);
  plan->kernel = p.kernel;
  plan->dv_tile = p.tile;
  plan->segments = p.P;
  plan->groups = p.ng;
  plan->state_split = p.sub;
  if (workspace_bytes) *workspace_bytes = L > 0 ? p.ws_bytes : 0;
  return LA_OK;
}

size_t la_chunk_fwd_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                                    int decay_kind) {
  if (check_chunk_shape(dtype, B, H, L, d_k, d_v, C) != LA_OK || L == 0) return 0;
  if (decay_kind < LA_DECAY_NONE || decay_kind > LA_DECAY_CHANNEL_LOG) return 0;
  // one size serves both forms: the larger of the two plans' workspaces
  const size_t plain = make_plan(B, H, L, d_k, d_v, C, dtype, decay_kind, false, nullptr).ws_bytes;
  const size_t normed = make_plan(B, H, L, d_k, d_v, C, dtype, decay_kind, true, nullptr).ws_bytes;
  return plain > normed ? plain : normed;
}

la_status la_state_init(float* state, int B, int H, int d_k, int d_v, void* stream) {
  if (B < 1 || H < 1) return LA_ERR_SHAPE;
  if (!dim_ok(d_k) || !dim_ok(d_v)) return LA_ERR_UNSUPPORTED;
  if (!state) return LA_ERR_NULL;
  if (!aligned(state, 16)) return LA_ERR_ALIGN;
  const size_t n = (size_t)B * H * d_k * d_v;
  return la::launch_fill_zero(state, n, as_stream(stream)) == hipSuccess ? LA_OK : LA_ERR_DEVICE;
}

}  // extern "C"

namespace {

la_status chunk_fwd_impl(const void* q, const void* k, const void* v, int dtype, int B, int H,
                         int L, int d_k, int d_v, int C, int phi, int decay_kind,
                         const float* decay_data, float* state, float* norm_state, bool norm,
                         const la_plan* request, void* out, void* workspace,
                         size_t workspace_bytes, void* stream, bool use_scratch = false) {
  la_status st = check_chunk_shape(dtype, B, H, L, d_k, d_v, C);
  if (st != LA_OK) return st;
  if (phi != LA_PHI_IDENTITY && phi != LA_PHI_ELU1) return LA_ERR_UNSUPPORTED;
  if (decay_kind < LA_DECAY_NONE || decay_kind > LA_DECAY_CHANNEL_LOG) return LA_ERR_UNSUPPORTED;
  st = check_request(request);
  if (st != LA_OK) return st;
  const Plan p = make_plan(B, H, L, d_k, d_v, C, dtype, decay_kind, norm, request);
  // bf16 inputs reach the normalised form and the per-channel decay through
  // the stripe kernel only, and not both at once
  const bool chan = decay_kind == LA_DECAY_CHANNEL_LOG;
  if ((norm || chan) && dtype == LA_BF16 && p.kernel != LA_KERNEL_STRIPE) return LA_ERR_UNSUPPORTED;
  if (norm && chan && dtype == LA_BF16) return LA_ERR_UNSUPPORTED;
  if (L == 0) return LA_OK;
  if (!q || !k || !v || !out) return LA_ERR_NULL;
  if (decay_kind != LA_DECAY_NONE && !decay_data) return LA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      (state && !aligned(state, 16)) || (norm_state && !aligned(norm_state, 16)) ||
      (decay_data && !aligned(decay_data, 4)))
    return LA_ERR_ALIGN;
  if (p.ws_bytes > 0) {
    if (use_scratch) {
      // la_chunk_fwd_noalloc: the device's fixed scratch array, if the plan fits it
      if (p.ws_bytes > kScratchBytes) return LA_ERR_WORKSPACE;
      workspace = device_scratch();
      workspace_bytes = kScratchBytes;
      if (!workspace) return LA_ERR_DEVICE;
    }
    if (!workspace || workspace_bytes < p.ws_bytes) return LA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return LA_ERR_ALIGN;
  }

  la::ChunkArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.state = state;
  a.decay = decay_kind == LA_DECAY_NONE ? nullptr : decay_data;
  a.B = B;
  a.H = H;
  a.L = L;
  a.DK = d_k;
  a.DV = d_v;
  a.C = C;
  a.phi = phi;
  a.decay_kind = decay_kind;
  a.tv = p.tv;
  a.ng = p.ng;
  a.n_v = d_v / p.tile;
  a.P = p.P;
  a.seg_chunks = p.seg_chunks;
  a.sub = p.sub;
  a.norm = norm ? 1 : 0;
  a.zstate = norm ? norm_state : nullptr;
  a.s0 = state;
  a.z0 = a.zstate;
  const hipStream_t s = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  // z_0 is read by every workgroup of a head and z_L written by one of them:
  // the workgroups read a copy
  if (p.copy_z0 && norm_state) {
    float* z0 = reinterpret_cast<float*>(ws + p.ws_z0_off);
    if (la::launch_copy_f32(z0, norm_state, (size_t)B * H * d_k, s) != hipSuccess)
      return LA_ERR_DEVICE;
    a.z0 = z0;
  }

  if (p.flags) a.ws_flag = reinterpret_cast<int*>(ws + p.ws_flag_off);
  if (p.copy_S0_host && state) {
    float* s0 = reinterpret_cast<float*>(ws + p.ws_S0_off);
    if (la::launch_copy_f32(s0, state, (size_t)B * H * d_k * d_v, s) != hipSuccess)
      return LA_ERR_DEVICE;
    a.s0 = s0;
  }

  hipError_t e;
  if (dtype == LA_F32) {
    a.n_units = B * H;
    e = la::launch_chunk_f32(a, s);
  } else {
    if (p.prefix) {
      a.ws_b = reinterpret_cast<float*>(ws + p.ws_b_off);
      e = la::launch_decay_prefix(a, s);
      if (e != hipSuccess) return LA_ERR_DEVICE;
    }
    if (p.P > 1) {
      a.ws_S = reinterpret_cast<float*>(ws + p.ws_S_off);
      a.ws_logA = reinterpret_cast<float*>(ws + p.ws_logA_off);
      a.ws_z = reinterpret_cast<float*>(ws + p.ws_z_off);
      // the state pass copies S_0 for the output pass, whose last segment
      // overwrites state with S_L
      a.ws_S0 = (p.copy_S0 && state) ? reinterpret_cast<float*>(ws + p.ws_S0_off) : nullptr;
      a.n_units = B * H * (p.P - 1) * p.sub;
      e = p.kernel == LA_KERNEL_STRIPE ? la::launch_chunk_stripe(a, /*state_only=*/true, s)
                                       : la::launch_chunk_bf16(a, /*state_only=*/true, s);
      if (e != hipSuccess) return LA_ERR_DEVICE;
      a.s0 = a.ws_S0;
      a.ws_S0 = nullptr;
    }
    a.n_units = B * H * p.P;
    e = p.kernel == LA_KERNEL_STRIPE ? la::launch_chunk_stripe(a, /*state_only=*/false, s)
                                     : la::launch_chunk_bf16(a, /*state_only=*/false, s);
  }
  return e == hipSuccess ? LA_OK : LA_ERR_DEVICE;
}

la_status decode_impl(const void* q, const void* k, const void* v, int dtype, int N, int H,
                      int d_k, int d_v, int phi, int decay_kind, const float* decay_data,
                      float* state, float* norm_state, bool norm, void* out, void* stream) {
  if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_UNSUPPORTED;
  if (N < 1 || H < 1) return LA_ERR_SHAPE;
  if (!dim_ok(d_k) || !dim_ok(d_v)) return LA_ERR_UNSUPPORTED;
  if (phi != LA_PHI_IDENTITY && phi != LA_PHI_ELU1) return LA_ERR_UNSUPPORTED;
  if (decay_kind < LA_DECAY_NONE || decay_kind > LA_DECAY_CHANNEL_LOG) return LA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !state || !out || (norm && !norm_state)) return LA_ERR_NULL;
  if (decay_kind != LA_DECAY_NONE && !decay_data) return LA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(state, 16) || (norm && !aligned(norm_state, 16)) ||
      (decay_data && !aligned(decay_data, 4)))
    return LA_ERR_ALIGN;
  la::DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.state = state;
  a.zstate = norm ? norm_state : nullptr;
  a.decay = decay_kind == LA_DECAY_NONE ? nullptr : decay_data;
  a.N = N;
  a.H = H;
  a.DK = d_k;
  a.DV = d_v;
  a.phi = phi;
  a.decay_kind = decay_kind;
  return la::launch_decode(a, dtype, as_stream(stream)) == hipSuccess ? LA_OK : LA_ERR_DEVICE;
}

}  // namespace

extern "C" {

la_status la_chunk_fwd(const void* q, const void* k, const void* v, int dtype, int B, int H,
                       int L, int d_k, int d_v, int C, int phi, int decay_kind,
                       const float* decay_data, float* state, void* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return chunk_fwd_impl(q, k, v, dtype, B, H, L, d_k, d_v, C, phi, decay_kind, decay_data, state,
                        nullptr, false, nullptr, out, workspace, workspace_bytes, stream);
}

la_status la_chunk_fwd_norm(const void* q, const void* k, const void* v, int dtype, int B, int H,
                            int L, int d_k, int d_v, int C, int phi, int decay_kind,
                            const float* decay_data, float* state, float* norm_state, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_fwd_impl(q, k, v, dtype, B, H, L, d_k, d_v, C, phi, decay_kind, decay_data, state,
                        norm_state, true, nullptr, out, workspace, workspace_bytes, stream);
}

la_status la_chunk_fwd_noalloc(const void* q, const void* k, const void* v, int dtype, int B,
                               int H, int L, int d_k, int d_v, int C, int phi, int decay_kind,
                               const float* decay_data, float* state, void* out, void* stream) {
  return chunk_fwd_impl(q, k, v, dtype, B, H, L, d_k, d_v, C, phi, decay_kind, decay_data, state,
                        nullptr, false, nullptr, out, nullptr, 0, stream, /*use_scratch=*/true);
}

la_status la_chunk_fwd_planned(const void* q, const void* k, const void* v, int dtype, int B,
                               int H, int L, int d_k, int d_v, int C, int phi, int decay_kind,
                               const float* decay_data, float* state, float* norm_state,
                               int normalize, const la_plan* plan, void* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return chunk_fwd_impl(q, k, v, dtype, B, H, L, d_k, d_v, C, phi, decay_kind, decay_data, state,
                        normalize ? norm_state : nullptr, normalize != 0, plan, out, workspace,
                        workspace_bytes, stream);
}

la_status la_decode_step(const void* q, const void* k, const void* v, int dtype, int N, int H,
                         int d_k, int d_v, int phi, int decay_kind, const float* decay_data,
                         float* state, void* out, void* stream) {
  return decode_impl(q, k, v, dtype, N, H, d_k, d_v, phi, decay_kind, decay_data, state, nullptr,
                     false, out, stream);
}

la_status la_decode_step_norm(const void* q, const void* k, const void* v, int dtype, int N,
                              int H, int d_k, int d_v, int phi, int decay_kind,
                              const float* decay_data, float* state, float* norm_state, void* out,
                              void* stream) {
  return decode_impl(q, k, v, dtype, N, H, d_k, d_v, phi, decay_kind, decay_data, state,
                     norm_state, true, out, stream);
}

}  // extern "C"

namespace {

// The delta rule's workspace: W and U0 (bf16 on the matrix-core path, fp32
// otherwise), then on the matrix-core path the chunks' bf16 score rows and
// the fp32 in-chunk decay prefix; byte offsets of U0, P and b, and the total.
struct DeltaWsLayout {
  size_t u_off = 0, p_off = 0, b_off = 0, bytes = 0;
};
DeltaWsLayout delta_ws_layout(int B, int H, int L, int d_k, int d_v, int C, int dtype) {
  const size_t ht = (size_t)B * H * L;
  const bool mfma = la::delta_uses_mfma(dtype, C, d_k, d_v);
  const size_t es = mfma ? 2 : sizeof(float);
  DeltaWsLayout w;
  w.u_off = round256(ht * d_k * es);
  size_t off = w.u_off + round256(ht * d_v * es);
  if (mfma) {
    w.p_off = off;
    off += round256(ht * la::kDeltaMaxC * 2);
    w.b_off = off;
    off += round256(ht * sizeof(float));
  }
  w.bytes = off;
  return w;
}
size_t delta_ws_bytes(int B, int H, int L, int d_k, int d_v, int C, int dtype) {
  return delta_ws_layout(B, H, L, d_k, d_v, C, dtype).bytes;
}

la_status check_delta_shape(int dtype, int B, int H, int L, int d_k, int d_v, int C) {
  const la_status st = check_chunk_shape(dtype, B, H, L, d_k, d_v, C);
  if (st != LA_OK) return st;
  if (C > la::kDeltaMaxC) return LA_ERR_UNSUPPORTED;
  return LA_OK;
}

}  // namespace

extern "C" {

size_t la_delta_fwd_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C, int dtype) {
  if (check_delta_shape(dtype, B, H, L, d_k, d_v, C) != LA_OK || L == 0) return 0;
  return delta_ws_bytes(B, H, L, d_k, d_v, C, dtype);
}

la_status la_delta_fwd(const void* q, const void* k, const void* v, const float* beta, int dtype,
                       int B, int H, int L, int d_k, int d_v, int C, int decay_kind,
                       const float* decay_data, float* state, void* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  la_status st = check_delta_shape(dtype, B, H, L, d_k, d_v, C);
  if (st != LA_OK) return st;
  if (decay_kind < LA_DECAY_NONE || decay_kind > LA_DECAY_TOKEN_GATE) return LA_ERR_UNSUPPORTED;
  if (L == 0) return LA_OK;
  if (!q || !k || !v || !beta || !out) return LA_ERR_NULL;
  if (decay_kind != LA_DECAY_NONE && !decay_data) return LA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      (state && !aligned(state, 16)) || !aligned(beta, 4) ||
      (decay_data && !aligned(decay_data, 4)))
    return LA_ERR_ALIGN;
  const size_t need = delta_ws_bytes(B, H, L, d_k, d_v, C, dtype);
  if (!workspace || workspace_bytes < need) return LA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return LA_ERR_ALIGN;
  la::DeltaArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.out = out;
  a.state = state;
  a.decay = decay_kind == LA_DECAY_NONE ? nullptr : decay_data;
  char* ws = static_cast<char*>(workspace);
  const DeltaWsLayout lay = delta_ws_layout(B, H, L, d_k, d_v, C, dtype);
  a.ws_W = reinterpret_cast<float*>(ws);
  a.ws_U = reinterpret_cast<float*>(ws + lay.u_off);
  if (la::delta_uses_mfma(dtype, C, d_k, d_v)) {
    a.ws_P = ws + lay.p_off;
    a.ws_b = reinterpret_cast<float*>(ws + lay.b_off);
  }
  a.B = B;
  a.H = H;
  a.L = L;
  a.DK = d_k;
  a.DV = d_v;
  a.C = C;
  a.decay_kind = decay_kind;
  a.dtype = dtype;
  return la::launch_delta(a, as_stream(stream)) == hipSuccess ? LA_OK : LA_ERR_DEVICE;
}

la_status la_delta_decode_step(const void* q, const void* k, const void* v, const float* beta,
                               int dtype, int N, int H, int d_k, int d_v, int decay_kind,
                               const float* decay_data, float* state, void* out, void* stream) {
  if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_UNSUPPORTED;
  if (N < 1 || H < 1) return LA_ERR_SHAPE;
  if (!dim_ok(d_k) || !dim_ok(d_v)) return LA_ERR_UNSUPPORTED;
  if (decay_kind < LA_DECAY_NONE || decay_kind > LA_DECAY_TOKEN_GATE) return LA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !beta || !state || !out) return LA_ERR_NULL;
  if (decay_kind != LA_DECAY_NONE && !decay_data) return LA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(state, 16) || !aligned(beta, 4) || (decay_data && !aligned(decay_data, 4)))
    return LA_ERR_ALIGN;
  la::DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.state = state;
  a.beta = beta;
  a.decay = decay_kind == LA_DECAY_NONE ? nullptr : decay_data;
  a.N = N;
  a.H = H;
  a.DK = d_k;
  a.DV = d_v;
  a.phi = LA_PHI_IDENTITY;
  a.decay_kind = decay_kind;
  return la::launch_decode(a, dtype, as_stream(stream)) == hipSuccess ? LA_OK : LA_ERR_DEVICE;
}

}  // extern "C"
