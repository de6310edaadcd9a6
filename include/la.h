/*
 * la.h -- C ABI of liblinattn.so: chunkwise causal linear attention on
 * AMD MI355X (gfx950).
 *
 * The operation (one head; every head of a [B, H] batch is independent):
 *
 *   S_t = a_t S_{t-1} + phi(k_t) v_t^T        S is d_k x d_v (rows = key dim)
 *   o_t = phi(q_t)^T S_t                      read after the write
 *
 * - The state, the outer-product write k v^T and the update-then-read order
 *   follow "Linear / Sparse Attention - minimal runnable implementation"
 *   (linear_attn_recurrent), whose chunkwise form (linear_attn_chunkwise) is
 *   what la_chunk_fwd computes: per chunk of C tokens, an inter-chunk term
 *   Q_c S_c, an intra-chunk term ((Q_c K_c^T) masked by tril incl. the
 *   diagonal) V_c, then S_{c+1} = S_c + K_c^T V_c; the last chunk may be short.
 * - The decay a_t follows CS336 lecture 4 code 1, section 4
 *   (gated_linear_attention_recurrent): S_t = gamma_t S_{t-1} + k_t v_t^T with
 *   gamma_t in (0, 1], constant per head (RetNet, tutorial section 2.4) or
 *   token dependent; the gated kind uses a_t = exp(-softplus(g_t)), the
 *   Mamba-style discretised decay exp(Delta A) with Delta = softplus(g) and
 *   A = -1 (tutorial sections 3.3 and 4.2).  The tutorial's section 6.2 says
 *   the chunkwise form folds the cumulative decay into S_c and the in-chunk
 *   mask; the library does so in log space, so every factor is exp(<= 0).
 * - phi is the identity or elu(x) + 1 with alpha = 1, applied to q and k,
 *   never to v ("adv13 -- Linear Attention / SSM", sections 3.1-4.3).
 * - No normaliser phi(q)^T z_t: this is the un-normalised form whose
 *   recurrent == chunkwise equivalence the tutorial's section 6.2 states.
 *
 * Conventions for every entry point
 * - Tensor pointers are DEVICE pointers (hipMalloc'd or torch tensors on the
 *   GPU), contiguous, row-major, 16-byte aligned.  The caller owns and frees
 *   all memory, including the workspace; the library allocates nothing.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *   and the call returns without synchronising.  Results are valid once the
 *   caller has synchronised that stream.
 * - Every argument is validated on the host before anything is launched, so
 *   a call that returns an error has not touched device memory.  Values that
 *   live on the device (decay parameters, NaN/Inf in inputs) are not
 *   checked: NaN and Inf propagate.
 * - Outputs must not alias inputs or the state (not checked).
 * - Calls are thread-safe; calls that share output buffers must be ordered
 *   by the caller.  The library's only global state is a cache of each
 *   device's compute-unit count, filled on first use.
 */
#ifndef LA_H_
#define LA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LA_OK = 0,
  LA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  LA_ERR_SHAPE = 2,       /* B, H or N < 1, L < 0, C < 1                         */
  LA_ERR_UNSUPPORTED = 3, /* d_k, d_v or C outside {16,32,64,128}; unknown enum  */
  LA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                    */
  LA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required            */
  LA_ERR_DEVICE = 6       /* a HIP call or kernel launch failed                  */
} la_status;

typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

typedef enum { LA_PHI_IDENTITY = 0, LA_PHI_ELU1 = 1 } la_phi;

typedef enum {
  LA_DECAY_NONE = 0,       /* a_t = 1; decay_data ignored (may be NULL)          */
  LA_DECAY_HEAD = 1,       /* a_t = gamma[h]; decay_data = float gamma[H], 0<gamma<=1 */
  LA_DECAY_TOKEN_LOG = 2,  /* a_t = exp(log_a[b,h,t]); decay_data = float [B,H,L], <= 0 */
  LA_DECAY_TOKEN_GATE = 3, /* a_t = exp(-softplus(g[b,h,t])); decay_data = float [B,H,L] */
  LA_DECAY_CHANNEL_LOG = 4 /* per key channel (GLA's diagonal gate, the tutorial's
                              section 2.4): S_t = diag(exp(log_a[b,h,t,:])) S_{t-1} + k v^T;
                              decay_data = float [B,H,L,d_k], <= 0 */
} la_decay_kind;

/*
 * la_state_init -- zero the recurrent state.
 *   state : float [B, H, d_k, d_v], device, written.
 * Errors: LA_ERR_NULL, LA_ERR_SHAPE (B or H < 1), LA_ERR_UNSUPPORTED (d_k, d_v),
 *         LA_ERR_ALIGN, LA_ERR_DEVICE.
 * A fill kernel (not hipMemsetAsync), so the call may be captured in a HIP graph.
 */
la_status la_state_init(float* state, int B, int H, int d_k, int d_v, void* stream);

/*
 * la_chunk_fwd_workspace_bytes -- bytes of device workspace la_chunk_fwd and
 * la_chunk_fwd_norm need for this problem (0 when none is needed): per-segment
 * state (and normaliser) increments and a copy of S_0 when the sequence is
 * split into segments, a copy of z_0 when the normalised form spreads a head
 * over several workgroups (the workgroup that writes S_L or z_L back may
 * finish before the others have read S_0 or z_0), and the in-chunk prefix
 * sums of log a (4 bytes per head-token) for the token-dependent decays.
 * Pure host function; returns 0 for arguments la_chunk_fwd would reject.
 */
size_t la_chunk_fwd_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                                    int decay_kind);

/*
 * la_chunk_fwd -- the chunkwise-parallel forward over a whole sequence.
 *
 *   q, k       : [B, H, L, d_k], dtype          (device, read)
 *   v          : [B, H, L, d_v], dtype          (device, read)
 *   dtype      : LA_F32 (fp32 in, fp32 arithmetic throughout) or
 *                LA_BF16 (bf16 in, bf16 matrix-core products, fp32 accumulation
 *                and fp32 state)
 *   C          : chunk size, one of 16, 32, 64, 128.  A performance knob only:
 *                the result does not depend on C beyond rounding.  C >= L means
 *                one chunk.  The requested C is honoured, never replaced.
 *   phi        : la_phi
 *   decay_kind : la_decay_kind; decay_data as described there (device, read).
 *                Any log decay <= 0 is taken, -inf included (a = 0: the step
 *                forgets).  LA_DECAY_CHANNEL_LOG on bf16 inputs: a chunk whose
 *                decay sums below 2^-192 in some channel makes its workgroup's
 *                segment be recomputed by an exact (slower) pass; the result
 *                is the same either way.  The token kinds take a per-token
 *                decay below 2^-126 (the smallest normal fp32) as 2^-126: any
 *                factor containing it is below the fp32 normal range either
 *                way.
 *   state      : float [B, H, d_k, d_v] (device) or NULL.  In: S_0; out: S_L.
 *                NULL means S_0 = 0 and the final state is dropped.
 *   out        : [B, H, L, d_v], same dtype as q (device, written)
 *   workspace  : device scratch of at least la_chunk_fwd_workspace_bytes(...)
 *                bytes (may be NULL when that is 0); contents need no
 *                initialisation and are garbage afterwards.
 * L == 0 is a no-op that returns LA_OK (the state is left as is).
 * Errors: LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_UNSUPPORTED, LA_ERR_ALIGN,
 *         LA_ERR_WORKSPACE, LA_ERR_DEVICE.
 */
la_status la_chunk_fwd(const void* q, const void* k, const void* v, int dtype, int B, int H,
                       int L, int d_k, int d_v, int C, int phi, int decay_kind,
                       const float* decay_data, float* state, void* out, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * la_decode_step -- one recurrent token for N sequences x H heads, in place on
 * the state (the recurrent form "linear_attn_recurrent" applied once; the
 * state a prefill left behind is the S_{t-1} of the first step).
 *
 *   q, k       : [N, H, d_k], dtype     v : [N, H, d_v], dtype   (device, read)
 *   decay_data : NULL | float gamma[H] | float [N, H] (this step's log a or g)
 *                | float [N, H, d_k] (LA_DECAY_CHANNEL_LOG: this step's log a)
 *   state      : float [N, H, d_k, d_v] (device, read and written; required)
 *   out        : [N, H, d_v], same dtype as q (device, written)
 * Errors: LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_UNSUPPORTED, LA_ERR_ALIGN, LA_ERR_DEVICE.
 */
la_status la_decode_step(const void* q, const void* k, const void* v, int dtype, int N, int H,
                         int d_k, int d_v, int phi, int decay_kind, const float* decay_data,
                         float* state, void* out, void* stream);

/*
 * la_chunk_fwd_norm -- the normalised form (the linear/sparse attention
 * tutorial, section 2.2, boxed recurrence):
 *
 *   S_t = a_t S_{t-1} + phi(k_t) v_t^T,   z_t = a_t z_{t-1} + phi(k_t),
 *   o_t = phi(q_t)^T S_t / phi(q_t)^T z_t
 *
 * z is carried chunkwise as one more value column of ones (tutorial section
 * 6.2).  Nothing is added to the denominator (the pages give no term); it
 * stays positive for phi = elu + 1 and positive initial z, and is otherwise
 * the caller's responsibility (a zero gives Inf/NaN).
 *   norm_state : [B,H,d_k] fp32 z; in: z_0, out: z_L.  NULL: z_0 = 0 and
 *                z_L is not written.  16-byte aligned.
 * Every other argument, the workspace size (la_chunk_fwd_workspace_bytes)
 * and the errors are those of la_chunk_fwd.  bf16 inputs need d_k, d_v >= 32
 * and C in {32, 64, 128} within the LDS and not LA_DECAY_CHANNEL_LOG (else
 * LA_ERR_UNSUPPORTED); fp32 inputs take every supported shape and decay.
 */
la_status la_chunk_fwd_norm(const void* q, const void* k, const void* v, int dtype, int B, int H,
                            int L, int d_k, int d_v, int C, int phi, int decay_kind,
                            const float* decay_data, float* state, float* norm_state, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * la_decode_step_norm -- one token of the normalised form for N x H heads:
 * S' = a S + phi(k) v^T, z' = a z + phi(k), o = phi(q)^T S' / phi(q)^T z'.
 *   norm_state : [N,H,d_k] fp32 z, updated in place (required).
 * Every other argument and the errors are those of la_decode_step.
 */
la_status la_decode_step_norm(const void* q, const void* k, const void* v, int dtype, int N,
                              int H, int d_k, int d_v, int phi, int decay_kind,
                              const float* decay_data, float* state, float* norm_state, void* out,
                              void* stream);

/* la_status_string -- a static, human-readable name for a status code. */
const char* la_status_string(int status);

/*
 * The delta rule (DeltaNet; with a scalar decay, Gated DeltaNet): "Linear /
 * Sparse Attention - minimal runnable implementation", delta_rule_recurrent,
 * and the linear/sparse attention tutorial, sections 5.1-5.3, Q15, Q17, Q23.
 * The pages' value-by-key state S' is stored transposed (S = S'^T, d_k x d_v,
 * row = key dim, like the linear-attention state), so per head and token
 *
 *   S_t = a_t (S_{t-1} - beta_t k_t (k_t^T S_{t-1})) + beta_t k_t v_t^T
 *   o_t = q_t^T S_t                                   (read after the write)
 *
 * Keys are used as given (the pages normalise them before the call; the
 * update is a contraction for unit keys and 0 <= beta <= 2).  No feature map.
 *
 * la_delta_fwd -- the chunkwise form over a [B,H,L] batch.  The chunk's erase
 * products are folded into a unit lower-triangular solve per chunk (the WY
 * idea of tutorial section 5.3): a chunk-parallel pass solves every chunk and
 * writes W = T diag(beta e^b) K and U0 = T diag(beta) V into the workspace
 * (for bf16 inputs with 64-token chunks as bf16, together with each chunk's
 * causal scores (q_i . k_j) e^{b_i - b_j}, j <= i, and its in-chunk decay
 * prefix b), then a sequential pass per head computes U = U0 - W S_c and the
 * decayed linear-attention chunk with V replaced by U.  Accumulation is fp32
 * (bf16 inputs: bf16 matrix-core products).
 *   q, k       : [B,H,L,d_k] (device, read), dtype LA_F32 or LA_BF16
 *   v          : [B,H,L,d_v] (device, read)
 *   beta       : [B,H,L] fp32 write strengths (device, read), 4-byte aligned
 *   C          : chunk length, 16, 32 or 64
 *   decay_kind : LA_DECAY_NONE, _HEAD, _TOKEN_LOG or _TOKEN_GATE with
 *                decay_data as for la_chunk_fwd (the per-channel kind is
 *                LA_ERR_UNSUPPORTED here)
 *   state      : [B,H,d_k,d_v] fp32 or NULL; in: S_0, out: S_L (NULL: S_0 = 0)
 *   out        : [B,H,L,d_v] of dtype (device, written)
 *   workspace  : device scratch of at least la_delta_fwd_workspace_bytes(),
 *                16-byte aligned, owned by the caller; contents undefined after
 *                (per head-token: 2 (d_k + d_v + 64) + 4 bytes for bf16 inputs
 *                with 64-token chunks, d_k >= 32 and d_v a multiple of 32,
 *                4 (d_k + d_v) otherwise; each region rounded up to 256 bytes)
 * Shapes, alignment and errors as for la_chunk_fwd (LA_ERR_NULL for a NULL
 * beta, LA_ERR_WORKSPACE for a missing or small workspace).  Asynchronous on
 * `stream`.
 */
size_t la_delta_fwd_workspace_bytes(int B, int H, int L, int d_k, int d_v, int C, int dtype);
la_status la_delta_fwd(const void* q, const void* k, const void* v, const float* beta, int dtype,
                       int B, int H, int L, int d_k, int d_v, int C, int decay_kind,
                       const float* decay_data, float* state, void* out, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * la_delta_decode_step -- one token of the delta rule for N sequences x H
 * heads: r = k^T S, S' = a (S - beta k r^T) + beta k v^T, o = q^T S'.
 *   beta       : [N,H] fp32 (device, read)
 *   decay_data : NULL | gamma[H] | [N,H] (this step's log a or g)
 * Every other argument and the errors are those of la_decode_step (phi is
 * the identity; the per-channel kind is LA_ERR_UNSUPPORTED).
 */
la_status la_delta_decode_step(const void* q, const void* k, const void* v, const float* beta,
                               int dtype, int N, int H, int d_k, int d_v, int decay_kind,
                               const float* decay_data, float* state, void* out, void* stream);

/*
 * la_chunk_fwd_noalloc -- la_chunk_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): no workspace argument, and the call allocates and
 * frees nothing.  The workspace la_chunk_fwd would take lives instead in a
 * fixed scratch array of LA_NOALLOC_SCRATCH_BYTES bytes in the library's
 * device memory, one per device, held from the library's load until the
 * process ends.  Every other argument, the result and the errors are those
 * of la_chunk_fwd; a problem whose workspace
 * (la_chunk_fwd_workspace_bytes) exceeds the scratch returns
 * LA_ERR_WORKSPACE before anything is launched, and LA_ERR_DEVICE means the
 * scratch's device address could not be looked up.  The scratch needs no
 * initialisation and keeps the last call's contents.  All calls on one
 * device share it: calls that may overlap on one device (other streams,
 * other threads) race and must be ordered by the caller.
 */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
la_status la_chunk_fwd_noalloc(const void* q, const void* k, const void* v, int dtype, int B,
                               int H, int L, int d_k, int d_v, int C, int phi, int decay_kind,
                               const float* decay_data, float* state, void* out, void* stream);

/*
 * Launch plan of la_chunk_fwd (for tests and benchmarks).  The library keeps
 * no plan state: a plan is requested per call.
 *   kernel    LA_KERNEL_F32 (fp32 inputs: one workgroup per head and 32-column
 *             tile), LA_KERNEL_STRIP (bf16: 16x16 MFMA, 4-wave column groups,
 *             any d_k, d_v, C) or LA_KERNEL_STRIPE (bf16: 32x32 MFMA, one
 *             wave per 32 value columns holding its part of the state in
 *             registers; d_k, d_v >= 32 and C >= 32).
 *   dv_tile   value columns one workgroup covers (16, 32, 64 or 128)
 *   segments  sequence segments per head (> 1: a state pass runs first)
 *   groups    strip kernel: 4-wave column groups per workgroup (1 or 2);
 *             stripe kernel: waves per 32-column stripe, each holding a
 *             share of the keys of the state (1 or 2; 2 needs d_k >= 64)
 *   state_split  state-pass workgroups per segment (segments > 1): each
 *             takes an equal share of the segment's chunks, and the output
 *             pass composes their (decay, increment) pairs like segments; a
 *             divisor of the segment's chunk count (a request is reduced to
 *             one), 1 with one segment
 * In a request, a field at 0 keeps the automatic choice.  The automatic plan
 * splits sequences into segments until the grid covers the current device's
 * compute units (queried once per device and cached; 256 when no device is
 * visible).  Requested values that do not fit a call are reduced to ones that
 * do (a stripe request the shape does not allow falls back to the strip
 * kernel).  fp32 inputs have one plan and ignore requests.  Results do not
 * depend on the plan beyond rounding; tests use requests to check that.
 */
typedef struct {
  int kernel;
  int dv_tile;
  int segments;
  int groups;
  int state_split;
} la_plan;

enum { LA_KERNEL_AUTO = 0, LA_KERNEL_STRIP = 1, LA_KERNEL_STRIPE = 2, LA_KERNEL_F32 = 3 };

/*
 * la_chunk_fwd_plan -- resolve a plan (host only, launches nothing).
 *   plan            in: the request (all zero: automatic); out: the plan
 *                   la_chunk_fwd_planned takes with that request for these
 *                   arguments (la_chunk_fwd / la_chunk_fwd_norm: all zero)
 *   normalize       0: la_chunk_fwd; 1: la_chunk_fwd_norm
 *   workspace_bytes NULL, or out: the workspace bytes that plan needs
 * Returns LA_OK, LA_ERR_NULL for a NULL plan, LA_ERR_UNSUPPORTED for an
 * invalid kernel, tile or group count, LA_ERR_SHAPE for a negative segment
 * count, or the error la_chunk_fwd would return for these shapes.
 */
la_status la_chunk_fwd_plan(int B, int H, int L, int d_k, int d_v, int C, int dtype,
                            int decay_kind, int normalize, la_plan* plan,
                            size_t* workspace_bytes);

/*
 * la_chunk_fwd_planned -- la_chunk_fwd (normalize = 0; norm_state ignored) or
 * la_chunk_fwd_norm (normalize = 1) with a requested plan (NULL or all zero:
 * automatic).  The workspace must hold what la_chunk_fwd_plan reports for the
 * same request.  Errors: those of la_chunk_fwd, plus those of
 * la_chunk_fwd_plan for an invalid request.
 */
la_status la_chunk_fwd_planned(const void* q, const void* k, const void* v, int dtype, int B,
                               int H, int L, int d_k, int d_v, int C, int phi, int decay_kind,
                               const float* decay_data, float* state, float* norm_state,
                               int normalize, const la_plan* plan, void* out, void* workspace,
                               size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LA_H_ */
