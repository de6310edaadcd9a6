"""fp64 CPU oracle for causal linear attention -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package.  It shares no code with the HIP library
under `chunkwise_recurrence_amd/` and never imports it.

Three independent ways to compute the same thing, each in float64:

* `recurrent`   -- the plain definition, token by token (C, `la_oracle.c`).
  This is THE oracle the GPU is compared with.
* `parallel`    -- the fully parallel masked form Y = ((Q K^T) o D) V with
  D[t,s] = prod_{r=s+1..t} a_r for s <= t and 0 above the diagonal
  (CS336 lecture 4 code 1, `causal_linear_attention_parallel` and
  `gated_linear_attention_parallel`, whose derivation expands the recurrence
  into exactly this sum).  Here D is built from explicit products, not from
  the log-space cumsum, so that it is a different computation path.
* `chunkwise`   -- the chunkwise form: per chunk, inter = diag(e^b) Q_c S_c,
  intra = ((Q_c K_c^T) o D_c) V_c, S_{c+1} = e^{b_last} S_c +
  (diag(e^{b_last - b}) K_c)^T V_c, with b the in-chunk inclusive cumsum of
  log a ("Linear / Sparse Attention" `linear_attn_chunkwise` for the
  undecayed skeleton; tutorial section 6.2 says decayed variants fold the
  cumulative decay into S_c and the in-chunk mask; the decayed formulas are
  obtained by expanding the recurrence over one chunk).

`parallel` and `chunkwise` exist to pin `recurrent` (they are never compared
with the GPU).  All three take the decay as a per-token multiplier array
`a` [.., L] produced by `decay_multipliers`, which turns the library's decay
parameters into a_t exactly as the pages define them.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

PHI_IDENTITY = 0
PHI_ELU1 = 1
DECAY_NONE = 0
DECAY_HEAD = 1
DECAY_LOG = 2
DECAY_GATE = 3
DECAY_CHANNEL = 4

_libs: dict = {}


def _load(path: str | None = None):
    path = LIB_PATH if path is None else path
    if path not in _libs:
        if path == LIB_PATH and not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(path)
        d = ctypes.POINTER(ctypes.c_double)
        lib.oracle_recurrent.restype = ctypes.c_int
        lib.oracle_recurrent.argtypes = [ctypes.c_int] * 5 + [d, d, d, ctypes.c_int, ctypes.c_int,
                                                             d, d, d, ctypes.c_int]
        lib.oracle_recurrent_norm.restype = ctypes.c_int
        lib.oracle_recurrent_norm.argtypes = [ctypes.c_int] * 5 + [
            d, d, d, ctypes.c_int, ctypes.c_int, d, d, d, d, ctypes.c_int]
        lib.oracle_delta.restype = ctypes.c_int
        lib.oracle_delta.argtypes = [ctypes.c_int] * 5 + [d, d, d, d, ctypes.c_int, d, d, d,
                                                         ctypes.c_int]
        _libs[path] = lib
    return _libs[path]


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def host_threads() -> int:
    """Host cores available to this process (sched_getaffinity)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# --------------------------------------------------------------------------
# the oracle proper
# --------------------------------------------------------------------------
def recurrent(q, k, v, phi: int = PHI_IDENTITY, decay_kind: int = DECAY_NONE, decay=None,
              state=None, nthreads: int | None = None, lib_path: str | None = None,
              normalize: bool = False, norm_state=None):
    """Token-by-token fp64 recurrence (`la_oracle.c`).

    q, k: [B,H,L,dk]; v: [B,H,L,dv]; decay: None | gamma[H] | log_a or g [B,H,L];
    state: [B,H,dk,dv] initial state (zeros if None).
    lib_path: another build of `la_oracle.c` to run instead of the default one
    (the tests use it to check that deliberately broken copies get caught).
    normalize: the normalised form o_t = phi(q_t)^T S_t / phi(q_t)^T z_t with
    z_t = a_t z_{t-1} + phi(k_t); norm_state: [B,H,dk] z_0 (zeros if None).
    Returns (out [B,H,L,dv], final state [B,H,dk,dv]) as float64 arrays, and
    the final z [B,H,dk] as a third element when normalize.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, H, L, dk) and v.shape == (B, H, L, dv)
    S = np.zeros((B, H, dk, dv)) if state is None else _f64(state).copy()
    assert S.shape == (B, H, dk, dv)
    out = np.zeros((B, H, L, dv))
    Z = None
    if normalize:
        Z = np.zeros((B, H, dk)) if norm_state is None else _f64(norm_state).copy()
        assert Z.shape == (B, H, dk)
    if decay_kind == DECAY_NONE:
        dec = np.zeros(1)
    elif decay_kind == DECAY_HEAD:
        dec = _f64(decay).reshape(H)
    elif decay_kind == DECAY_CHANNEL:
        dec = _f64(decay).reshape(B, H, L, dk)
    else:
        dec = _f64(decay).reshape(B, H, L)
    if B * H == 0 or L == 0:
        return (out, S, Z) if normalize else (out, S)
    n = host_threads() if nthreads is None else nthreads
    if normalize:
        _load(lib_path).oracle_recurrent_norm(B, H, L, dk, dv, _ptr(q), _ptr(k), _ptr(v), phi,
                                              decay_kind, _ptr(dec), _ptr(S), _ptr(Z),
                                              _ptr(out), n)
        return out, S, Z
    _load(lib_path).oracle_recurrent(B, H, L, dk, dv, _ptr(q), _ptr(k), _ptr(v), phi,
                                     decay_kind, _ptr(dec), _ptr(S), _ptr(out), n)
    return out, S


def decode_step(q, k, v, phi: int = PHI_IDENTITY, decay_kind: int = DECAY_NONE, decay=None,
                state=None, lib_path: str | None = None, normalize: bool = False,
                norm_state=None):
    """One recurrent step for N sequences x H heads: the same definition with L = 1.

    q, k: [N,H,dk]; v: [N,H,dv]; decay: None | gamma[H] | [N,H]; state [N,H,dk,dv];
    norm_state [N,H,dk] (normalised form).
    Returns (o [N,H,dv], new state) (+ new z when normalize).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, H, _ = q.shape
    dec = decay
    if decay_kind in (DECAY_LOG, DECAY_GATE):
        dec = _f64(decay).reshape(N, H, 1)
    elif decay_kind == DECAY_CHANNEL:
        dec = _f64(decay).reshape(N, H, 1, -1)
    r = recurrent(q[:, :, None, :], k[:, :, None, :], v[:, :, None, :], phi, decay_kind,
                  dec, state, lib_path=lib_path, normalize=normalize, norm_state=norm_state)
    return (r[0][:, :, 0, :],) + tuple(r[1:])


# --------------------------------------------------------------------------
# helpers shared by the two pinning forms below (not used by `recurrent`)
# --------------------------------------------------------------------------
def feature_map(x, phi: int) -> np.ndarray:
    """phi(x) = elu(x) + 1 (alpha = 1) or the identity, in fp64."""
    x = _f64(x)
    if phi == PHI_ELU1:
        return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    return x


def decay_multipliers(B: int, H: int, L: int, decay_kind: int, decay) -> np.ndarray:
    """a_t for every (b, h, t) as fp64 [B,H,L] (1 for no decay); [B,H,L,dk] for
    the per-channel kind."""
    if decay_kind == DECAY_CHANNEL:
        return np.exp(_f64(decay))
    if decay_kind == DECAY_NONE:
        return np.ones((B, H, L))
    if decay_kind == DECAY_HEAD:
        g = _f64(decay).reshape(1, H, 1)
        return np.broadcast_to(g, (B, H, L)).copy()
    x = _f64(decay).reshape(B, H, L)
    if decay_kind == DECAY_LOG:
        return np.exp(x)
    # exp(-softplus(g)) = 1 / (1 + e^g), evaluated without overflow
    return np.exp(-(np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))))


def parallel(q, k, v, a, phi: int = PHI_IDENTITY, state=None, normalize: bool = False,
             norm_state=None):
    """Fully parallel masked form, one [L,L] product per head (O(L^2)).

    o_t = sum_{s<=t} D[t,s] (phi(q_t).phi(k_s)) v_s + (prod_{r<=t} a_r) phi(q_t)^T S_0,
    D[t,s] = prod_{r=s+1..t} a_r (an explicit running product, no logs).
    Returns (out, final state) with S_L = sum_s D[L-1,s] phi(k_s) v_s^T + prod(a) S_0.
    normalize: every row is divided by the same masked sum with v replaced by
    ones, sum_{s<=t} D[t,s] (phi(q_t).phi(k_s)) + (prod_{r<=t} a_r) phi(q_t).z_0.
    """
    fq, fk, v, a = feature_map(q, phi), feature_map(k, phi), _f64(v), _f64(a)
    B, H, L, dk = fq.shape
    dv = v.shape[-1]
    S0 = np.zeros((B, H, dk, dv)) if state is None else _f64(state)
    out = np.zeros((B, H, L, dv))
    SL = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            D = np.zeros((L, L))
            for s in range(L):
                p = 1.0
                D[s, s] = 1.0
                for t in range(s + 1, L):
                    p *= a[b, h, t]
                    D[t, s] = p
            head = np.cumprod(a[b, h])  # prod_{r<=t} a_r: decay of S_0 seen at token t
            scores = fq[b, h] @ fk[b, h].T
            out[b, h] = (scores * D) @ v[b, h] + head[:, None] * (fq[b, h] @ S0[b, h])
            if normalize:
                z0 = np.zeros(dk) if norm_state is None else _f64(norm_state)[b, h]
                den = (scores * D).sum(axis=1) + head * (fq[b, h] @ z0)
                out[b, h] = out[b, h] / den[:, None]
            if L:
                SL[b, h] = (fk[b, h] * D[L - 1][:, None]).T @ v[b, h] + head[-1] * S0[b, h]
            else:
                SL[b, h] = S0[b, h]
    return out, SL


def chunk_spans(L: int, C: int):
    """(first, stop) token indices of the chunks of C tokens covering 0..L-1; the
    last span is shorter when C does not divide L."""
    firsts = np.arange(0, L, C, dtype=np.int64)
    stops = np.minimum(firsts + C, L)
    return list(zip(firsts.tolist(), stops.tolist()))


def _decayed_chunk(carry, Qc, Kc, Vc, log_ac, dtype):
    """One chunk of the decayed chunkwise form.  carry: the [dk, dv'] state on
    entry (dv' = dv, or dv + 1 with z as the last column).  Returns the chunk's
    rows of the numerator and the carry on exit."""
    cum = np.cumsum(log_ac).astype(dtype)           # b_i, inclusive, local to the chunk
    n = cum.shape[0]
    causal = np.tri(n, dtype=bool)                  # j <= i, diagonal included
    gaps = np.where(causal, cum[:, None] - cum[None, :], 0.0)
    weights = np.where(causal, np.exp(gaps), 0.0).astype(dtype)
    rows = np.exp(cum)[:, None] * (Qc @ carry) + ((Qc @ Kc.T) * weights) @ Vc
    tail = np.exp(cum[-1] - cum)                    # e^{b_last - b_j}
    carry = np.exp(cum[-1]) * carry + (Kc * tail[:, None]).T @ Vc
    return rows, carry


def chunkwise(q, k, v, a, C: int, phi: int = PHI_IDENTITY, state=None, dtype=np.float64,
              normalize: bool = False, norm_state=None):
    """Chunkwise form with decay folded in (log-space, every factor exp(<= 0)).

    Per chunk of c <= C tokens with b = inclusive cumsum of log a inside the chunk:
      O_c     = diag(e^b) Q_c S_c + ((Q_c K_c^T) o D_c) V_c,  D_c[i,j] = e^{b_i - b_j} [j <= i]
      S_{c+1} = e^{b_last} S_c + (diag(e^{b_last - b}) K_c)^T V_c
    ("Linear / Sparse Attention" `linear_attn_chunkwise` gives the undecayed
    form; the tutorial's section 6.2 says the decay folds into S_c and the
    in-chunk mask; the formulas come from expanding the recurrence over one
    chunk.)  A ragged last chunk simply has c < C rows.
    `dtype` is the working precision (float64 by default; float32 reproduces
    the magnitude of rounding error the pages print for their fp32 run).
    normalize: z is carried as one more value column of ones (the tutorial's
    section 6.2 suggestion), and every output row is divided by its entry.
    """
    fq, fk = feature_map(q, phi).astype(dtype), feature_map(k, phi).astype(dtype)
    v, a = _f64(v).astype(dtype), _f64(a)
    B, H, L, dk = fq.shape
    dv = v.shape[-1]
    S0 = np.zeros((B, H, dk, dv)) if state is None else _f64(state)
    z0 = np.zeros((B, H, dk)) if norm_state is None else _f64(norm_state)
    width = dv + 1 if normalize else dv
    out = np.zeros((B, H, L, dv), dtype)
    S_fin = np.zeros((B, H, dk, dv), dtype)
    Z_fin = np.zeros((B, H, dk), dtype) if normalize else None
    with np.errstate(divide="ignore"):
        log_a = np.log(a)
    spans = chunk_spans(L, C)
    for bh in np.ndindex(B, H):
        # the value columns, with a column of ones appended for z
        vals = np.concatenate([v[bh], np.ones((L, 1), dtype)], axis=1) if normalize else v[bh]
        carry = np.zeros((dk, width), dtype)
        carry[:, :dv] = S0[bh]
        if normalize:
            carry[:, dv] = z0[bh]
        for first, stop in spans:
            rows, carry = _decayed_chunk(carry, fq[bh][first:stop], fk[bh][first:stop],
                                         vals[first:stop], log_a[bh][first:stop], dtype)
            out[bh][first:stop] = rows[:, :dv] / rows[:, dv:] if normalize else rows
        S_fin[bh] = carry[:, :dv]
        if normalize:
            Z_fin[bh] = carry[:, dv]
    return (out, S_fin, Z_fin) if normalize else (out, S_fin)


def rel_err(x, ref) -> float:
    """max|x - ref| / max|ref| (the pages' 'max relative difference')."""
    x, ref = _f64(x), _f64(ref)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(x - ref)) if ref.size else 0.0
    return float(num / den) if den > 0 else float(num)


# --------------------------------------------------------------------------
# the per-channel (GLA) gate: S_t = diag(alpha_t) S_{t-1} + k_t v_t^T
# (linear/sparse attention tutorial, section 2.4)
# --------------------------------------------------------------------------
def parallel_channel(q, k, v, a, phi: int = PHI_IDENTITY, state=None, normalize: bool = False,
                     norm_state=None):
    """Fully parallel form of the per-channel gate with explicit products.

    a: [B,H,L,dk] multipliers.  o_t = sum_{s<=t} sum_d phi(q)_td phi(k)_sd
    D[t,s,d] v_s + sum_d phi(q)_td (prod_{r<=t} a_rd) S_0[d,:],
    D[t,s,d] = prod_{r=s+1..t} a_rd; S_L[d,:] = sum_s D[L-1,s,d] phi(k)_sd v_s
    + prod_r a_rd S_0[d,:].
    normalize: each row is divided by the same masked sum with v replaced by
    ones, sum_{s<=t} sum_d phi(q)_td phi(k)_sd D[t,s,d] + sum_d phi(q)_td
    (prod_{r<=t} a_rd) z_0[d] (the tutorial's section 2.2 boxed recurrence,
    with the diagonal gate of section 2.4 acting on z as on each row of S).
    """
    fq, fk, v, a = feature_map(q, phi), feature_map(k, phi), _f64(v), _f64(a)
    B, H, L, dk = fq.shape
    dv = v.shape[-1]
    S0 = np.zeros((B, H, dk, dv)) if state is None else _f64(state)
    out = np.zeros((B, H, L, dv))
    SL = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            D = np.zeros((L, L, dk))
            for s in range(L):
                p = np.ones(dk)
                D[s, s] = 1.0
                for t in range(s + 1, L):
                    p = p * a[b, h, t]
                    D[t, s] = p
            head = np.cumprod(a[b, h], axis=0)  # [L, dk]
            scores = np.einsum("td,sd,tsd->ts", fq[b, h], fk[b, h], D)
            out[b, h] = scores @ v[b, h] + (fq[b, h] * head) @ S0[b, h]
            if normalize:
                z0 = np.zeros(dk) if norm_state is None else _f64(norm_state)[b, h]
                den = scores.sum(axis=1) + (fq[b, h] * head) @ z0
                out[b, h] = out[b, h] / den[:, None]
            if L:
                SL[b, h] = (fk[b, h] * D[L - 1]).T @ v[b, h] + head[-1][:, None] * S0[b, h]
            else:
                SL[b, h] = S0[b, h]
    return out, SL


def _channel_chunk(carry, Qc, Kc, Vc, log_ac):
    """One chunk of the per-channel gate.  carry: [dk, dv'] on entry.  With
    cum[i, d] the in-chunk inclusive cumsum of log a per channel:
      rows  = (Q_c o e^{cum}) carry + P V_c,  P[i,j] = [j<=i] sum_d q_id k_jd e^{cum_id - cum_jd}
      carry = diag(e^{cum_last}) carry + (K_c o e^{cum_last - cum})^T V_c
    (every exponent <= 0)."""
    cum = np.cumsum(log_ac, axis=0)                   # [c, dk]
    n = cum.shape[0]
    causal = np.tri(n, dtype=bool)
    gaps = np.where(causal[..., None], cum[:, None, :] - cum[None, :, :], 0.0)
    P = np.where(causal, np.einsum("id,jd,ijd->ij", Qc, Kc, np.exp(gaps)), 0.0)
    rows = (Qc * np.exp(cum)) @ carry + P @ Vc
    carry = np.exp(cum[-1])[:, None] * carry + (Kc * np.exp(cum[-1] - cum)).T @ Vc
    return rows, carry


def chunkwise_channel(q, k, v, log_a, C: int, phi: int = PHI_IDENTITY, state=None,
                      normalize: bool = False, norm_state=None):
    """Chunkwise form of the per-channel gate (see `_channel_chunk`), chunk
    after chunk.  normalize: z rides along as one more value column of ones
    (tutorial section 6.2), decayed per channel like every row of S."""
    fq, fk, v, la = feature_map(q, phi), feature_map(k, phi), _f64(v), _f64(log_a)
    B_, H, L, dk = fq.shape
    dv = v.shape[-1]
    S0 = np.zeros((B_, H, dk, dv)) if state is None else _f64(state)
    z0 = np.zeros((B_, H, dk)) if norm_state is None else _f64(norm_state)
    out = np.zeros((B_, H, L, dv))
    S_fin = np.zeros((B_, H, dk, dv))
    Z_fin = np.zeros((B_, H, dk)) if normalize else None
    spans = chunk_spans(L, C)
    for bh in np.ndindex(B_, H):
        vals = np.concatenate([v[bh], np.ones((L, 1))], axis=1) if normalize else v[bh]
        carry = np.concatenate([S0[bh], z0[bh][:, None]], axis=1) if normalize else S0[bh].copy()
        for first, stop in spans:
            rows, carry = _channel_chunk(carry, fq[bh][first:stop], fk[bh][first:stop],
                                         vals[first:stop], la[bh][first:stop])
            out[bh][first:stop] = rows[:, :dv] / rows[:, dv:] if normalize else rows
        S_fin[bh] = carry[:, :dv]
        if normalize:
            Z_fin[bh] = carry[:, dv]
    return (out, S_fin, Z_fin) if normalize else (out, S_fin)


# --------------------------------------------------------------------------
# the delta rule (DeltaNet; Gated DeltaNet with a scalar decay a_t)
# ("Linear / Sparse Attention", delta_rule_recurrent; the tutorial, section
# 5.1-5.3, Q15, Q17, Q23)
# --------------------------------------------------------------------------
def delta_recurrent(q, k, v, beta, decay_kind: int = DECAY_NONE, decay=None, state=None,
                    nthreads: int | None = None, lib_path: str | None = None):
    """Token-by-token fp64 delta rule (`la_oracle.c`, oracle_delta): THE oracle
    the GPU's delta path is compared with.

    S_t = a_t (S_{t-1} - beta_t k_t (k_t^T S_{t-1})) + beta_t k_t v_t^T,
    o_t = q_t^T S_t; S is [dk, dv] (the transpose of the pages' value-by-key
    state).  q, k: [B,H,L,dk]; v: [B,H,L,dv]; beta: [B,H,L];
    decay: None | gamma[H] | log_a or g [B,H,L].  Returns (out, final state).
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, H, L, dk) and v.shape == (B, H, L, dv) and beta.shape == (B, H, L)
    S = np.zeros((B, H, dk, dv)) if state is None else _f64(state).copy()
    assert S.shape == (B, H, dk, dv)
    out = np.zeros((B, H, L, dv))
    assert decay_kind in (DECAY_NONE, DECAY_HEAD, DECAY_LOG, DECAY_GATE)
    if decay_kind == DECAY_NONE:
        dec = np.zeros(1)
    elif decay_kind == DECAY_HEAD:
        dec = _f64(decay).reshape(H)
    else:
        dec = _f64(decay).reshape(B, H, L)
    if B * H == 0 or L == 0:
        return out, S
    n = host_threads() if nthreads is None else nthreads
    _load(lib_path).oracle_delta(B, H, L, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                 decay_kind, _ptr(dec), _ptr(S), _ptr(out), n)
    return out, S


def delta_decode_step(q, k, v, beta, decay_kind: int = DECAY_NONE, decay=None, state=None,
                      lib_path: str | None = None):
    """One delta-rule step for N sequences x H heads (L = 1 of the recurrence).
    q, k: [N,H,dk]; v: [N,H,dv]; beta: [N,H]; decay: None | gamma[H] | [N,H]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, H, _ = q.shape
    dec = decay
    if decay_kind in (DECAY_LOG, DECAY_GATE):
        dec = _f64(decay).reshape(N, H, 1)
    out, S = delta_recurrent(q[:, :, None, :], k[:, :, None, :], v[:, :, None, :],
                             _f64(beta).reshape(N, H, 1), decay_kind, dec, state,
                             lib_path=lib_path)
    return out[:, :, 0, :], S


def delta_explicit(q, k, v, beta, a, state=None):
    """The delta rule as the pages write it, with explicit matrices: a value-by-key
    state S'_t = a_t S'_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T and
    o_t = S'_t q_t, then transposed back to the [dk, dv] orientation.
    a: [B,H,L] multipliers (decay_multipliers).  A separate computation path
    (full d_k x d_k products, the other orientation) that pins `delta_recurrent`.
    """
    q, k, v, beta, a = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(a)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    S0 = np.zeros((B, H, dk, dv)) if state is None else _f64(state)
    out = np.zeros((B, H, L, dv))
    SL = np.zeros((B, H, dk, dv))
    eye = np.eye(dk)
    for b in range(B):
        for h in range(H):
            Sp = S0[b, h].T.copy()  # [dv, dk]
            for t in range(L):
                kt = k[b, h, t]
                Sp = a[b, h, t] * Sp @ (eye - beta[b, h, t] * np.outer(kt, kt)) \
                    + beta[b, h, t] * np.outer(v[b, h, t], kt)
                out[b, h, t] = Sp @ q[b, h, t]
            SL[b, h] = Sp.T
    return out, SL


def _delta_chunk(carry, Qc, Kc, Vc, beta_c, log_ac):
    """One chunk of the delta rule's chunkwise form (see `delta_chunkwise`)."""
    cum = np.cumsum(log_ac)
    n = cum.shape[0]
    below = np.tri(n, dtype=bool)
    G = np.exp(np.where(below, cum[:, None] - cum[None, :], -np.inf))   # 0 above the diagonal
    system = np.eye(n) + beta_c[:, None] * (np.tril(Kc @ Kc.T, -1) * G)
    rhs = beta_c[:, None] * (Vc - np.exp(cum)[:, None] * (Kc @ carry))
    U = np.linalg.solve(system, rhs)
    rows = np.exp(cum)[:, None] * (Qc @ carry) + ((Qc @ Kc.T) * G) @ U
    carry = np.exp(cum[-1]) * carry + (np.exp(cum[-1] - cum)[:, None] * Kc).T @ U
    return rows, carry


def delta_chunkwise(q, k, v, beta, log_a, C: int, state=None):
    """Chunkwise (WY / UT) form of the delta rule, derived by unrolling the
    recurrence over one chunk (the tutorial's section 5.3 and Q23 give the
    idea -- the chunk's product of (I - beta k k^T) factors in a compact WY
    form -- but no steps).  Writing S_t = a_t S_{t-1} + k_t u_t^T with
    u_t = beta_t (v_t - a_t S_{t-1}^T k_t), and b the in-chunk inclusive
    cumsum of log a, the chunk's u's solve the unit lower-triangular system

      (I + diag(beta) (tril(K K^T, -1) o G)) U = diag(beta) (V - diag(e^b) K S_c),
      G[i,j] = e^{b_i - b_j},

    and then O_c = diag(e^b) Q S_c + ((Q K^T) o D) U with D = tril(G) (diagonal
    included) and S_{c+1} = e^{b_last} S_c + (diag(e^{b_last - b}) K)^T U.
    log_a: [B,H,L] (zeros for no decay).  fp64; np.linalg.solve for the system.
    """
    q, k, v, beta, la = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(log_a)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    S0 = np.zeros((B, H, dk, dv)) if state is None else _f64(state)
    out = np.zeros((B, H, L, dv))
    S_fin = np.zeros((B, H, dk, dv))
    spans = chunk_spans(L, C)
    for bh in np.ndindex(B, H):
        carry = S0[bh].copy()
        for first, stop in spans:
            out[bh][first:stop], carry = _delta_chunk(
                carry, q[bh][first:stop], k[bh][first:stop], v[bh][first:stop],
                beta[bh][first:stop], la[bh][first:stop])
        S_fin[bh] = carry
    return out, S_fin
