"""ctypes binding over liblinattn.so (include/la.h).

Argument marshalling only: torch tensors supply device pointers, shapes and
the current HIP stream; every step of the computation runs in the library's
kernels.  There is no fallback: a missing library or a failed call raises.
"""
from __future__ import annotations

import contextlib
import contextvars
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liblinattn.so")

LA_F32, LA_BF16 = 0, 1
PHI_IDENTITY, PHI_ELU1 = 0, 1
DECAY_NONE, DECAY_HEAD, DECAY_LOG, DECAY_GATE, DECAY_CHANNEL = 0, 1, 2, 3, 4
KERNEL_AUTO, KERNEL_STRIP, KERNEL_STRIPE, KERNEL_F32 = 0, 1, 2, 3


class Plan(ctypes.Structure):
    """la_plan: kernel, value columns per workgroup, segments, column groups, state-pass
    workgroups per segment."""
    _fields_ = [("kernel", ctypes.c_int), ("dv_tile", ctypes.c_int),
                ("segments", ctypes.c_int), ("groups", ctypes.c_int),
                ("state_split", ctypes.c_int)]

    def as_tuple(self):
        return (self.kernel, self.dv_tile, self.segments, self.groups, self.state_split)

# every symbol include/la.h declares
EXPORTS = ("la_state_init", "la_chunk_fwd_workspace_bytes", "la_chunk_fwd", "la_decode_step",
           "la_status_string", "la_chunk_fwd_plan", "la_chunk_fwd_planned", "la_chunk_fwd_norm",
           "la_decode_step_norm", "la_delta_fwd_workspace_bytes", "la_delta_fwd",
           "la_delta_decode_step", "la_chunk_fwd_noalloc")
# size of the fixed scratch array la_chunk_fwd_noalloc uses (LA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20

_lib = None
# the plan request chunk_fwd passes when given none (tests use `using_plan`);
# a context variable, so threads and tasks each see their own
_PLAN_REQUEST: contextvars.ContextVar = contextvars.ContextVar("la_plan_request", default=None)


class LAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load liblinattn.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m chunkwise_recurrence_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p
    lib.la_state_init.restype = i
    lib.la_state_init.argtypes = [vp, i, i, i, i, vp]
    lib.la_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.la_chunk_fwd_workspace_bytes.argtypes = [i] * 8
    lib.la_chunk_fwd.restype = i
    lib.la_chunk_fwd.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, i, f, vp, vp, vp,
                                 ctypes.c_size_t, vp]
    lib.la_decode_step.restype = i
    lib.la_decode_step.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, vp]
    lib.la_chunk_fwd_norm.restype = i
    lib.la_chunk_fwd_norm.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, i, f, vp, vp, vp, vp,
                                      ctypes.c_size_t, vp]
    lib.la_decode_step_norm.restype = i
    lib.la_decode_step_norm.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, vp, vp]
    lib.la_delta_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.la_delta_fwd_workspace_bytes.argtypes = [i] * 7
    lib.la_delta_fwd.restype = i
    lib.la_delta_fwd.argtypes = [vp, vp, vp, f, i, i, i, i, i, i, i, i, f, vp, vp, vp,
                                 ctypes.c_size_t, vp]
    lib.la_delta_decode_step.restype = i
    lib.la_delta_decode_step.argtypes = [vp, vp, vp, f, i, i, i, i, i, i, f, vp, vp, vp]
    lib.la_chunk_fwd_noalloc.restype = i
    lib.la_chunk_fwd_noalloc.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, i, f, vp, vp, vp]
    lib.la_status_string.restype = ctypes.c_char_p
    lib.la_status_string.argtypes = [i]
    lib.la_chunk_fwd_plan.restype = i
    lib.la_chunk_fwd_plan.argtypes = [i] * 9 + [ctypes.POINTER(Plan),
                                                ctypes.POINTER(ctypes.c_size_t)]
    lib.la_chunk_fwd_planned.restype = i
    lib.la_chunk_fwd_planned.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, i, f, vp, vp, i,
                                         ctypes.POINTER(Plan), vp, vp, ctypes.c_size_t, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().la_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LA_F32
    if t.dtype == torch.bfloat16:
        return LA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t: torch.Tensor, name: str, shape: tuple, dtype: torch.dtype):
    """Raise unless t has exactly this shape and dtype (the C ABI sees only pointers, so a
    wrong-sized buffer would be read or written out of bounds)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _decay_shape(decay_kind: int, B: int, H: int, L: int, dk: int):
    """Shape of the decay data la_chunk_fwd reads for this kind (None: no data)."""
    return {DECAY_NONE: None, DECAY_HEAD: (H,), DECAY_LOG: (B, H, L), DECAY_GATE: (B, H, L),
            DECAY_CHANNEL: (B, H, L, dk)}.get(decay_kind, "bad")


def _check_decay(decay, decay_kind: int, B: int, H: int, L: int, dk: int, kinds=None):
    shape = _decay_shape(decay_kind, B, H, L, dk)
    if shape == "bad" or (kinds is not None and decay_kind not in kinds):
        raise ValueError(f"unsupported decay kind {decay_kind}")
    if shape is None:
        return None  # ignored by the library
    if decay is None:
        raise ValueError(f"decay kind {decay_kind} needs decay data of shape {shape}")
    _shape(decay, "decay", shape, torch.float32)
    return decay


def _check_workspace(workspace, need: int):
    if workspace is None:
        return
    if workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(status: int, where: str):
    if status != 0:
        raise LAError(status, where)


def _request(plan_request):
    """A Plan request from a tuple / Plan / None (None: the context's request, if any)."""
    r = _PLAN_REQUEST.get() if plan_request is None else plan_request
    if r is None:
        return None
    if isinstance(r, Plan):
        return Plan(*r.as_tuple())
    r = tuple(int(x) for x in r)
    if len(r) > 5:
        raise ValueError("a plan request has at most 5 fields")
    return Plan(*(r + (0,) * (5 - len(r))))


@contextlib.contextmanager
def using_plan(kernel: int = 0, dv_tile: int = 0, segments: int = 0, groups: int = 0,
               state_split: int = 0):
    """Within the block, chunk_fwd and plan() request this launch plan (0 = automatic) unless
    given one explicitly.  Per thread / task: the library itself keeps no plan state."""
    token = _PLAN_REQUEST.set((int(kernel), int(dv_tile), int(segments), int(groups),
                               int(state_split)))
    try:
        yield
    finally:
        _PLAN_REQUEST.reset(token)


def _resolve(B, H, L, dk, dv, C, dtype, decay_kind, normalize, plan_request):
    p = _request(plan_request) or Plan()
    ws = ctypes.c_size_t(0)
    _check(load().la_chunk_fwd_plan(B, H, L, dk, dv, C, dtype, decay_kind, int(bool(normalize)),
                                    ctypes.byref(p), ctypes.byref(ws)), "la_chunk_fwd_plan")
    return p, int(ws.value)


def plan(B: int, H: int, L: int, dk: int, dv: int, C: int, dtype: int = LA_BF16,
         decay_kind: int = DECAY_NONE, normalize: bool = False, request=None):
    """(kernel, value columns per workgroup, segments per head, column groups, state-pass
    workgroups per segment) of the forward."""
    p, _ = _resolve(B, H, L, dk, dv, C, dtype, decay_kind, normalize, request)
    return p.as_tuple()


def plan_workspace_bytes(B: int, H: int, L: int, dk: int, dv: int, C: int, dtype: int = LA_BF16,
                         decay_kind: int = DECAY_NONE, normalize: bool = False,
                         request=None) -> int:
    """Workspace bytes the forward needs with this plan request (or the context's)."""
    return _resolve(B, H, L, dk, dv, C, dtype, decay_kind, normalize, request)[1]


def chunk_fwd_workspace_bytes(B: int, H: int, L: int, dk: int, dv: int, C: int,
                              dtype: int = LA_BF16, decay_kind: int = DECAY_NONE) -> int:
    return int(load().la_chunk_fwd_workspace_bytes(B, H, L, dk, dv, C, dtype, decay_kind))


def state_init(state: torch.Tensor, stream=None) -> torch.Tensor:
    """Zero a [B,H,dk,dv] fp32 state on the device."""
    _dev(state, "state")
    if state.dtype != torch.float32 or state.dim() != 4:
        raise ValueError("state must be float32 [B,H,dk,dv]")
    B, H, dk, dv = state.shape
    _check(load().la_state_init(_ptr(state), B, H, dk, dv, _stream(stream)), "la_state_init")
    return state


def _qkv(q, k, v, lead: int):
    """Shapes of q, k, v ([..., L, dk] / [..., L, dv] with `lead` leading dims)."""
    if q.dim() != lead + 1 or k.dim() != lead + 1 or v.dim() != lead + 1:
        raise ValueError(f"q, k, v must have {lead + 1} dimensions")
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1]:
        raise ValueError("q, k must share a shape and v must match them but for its last dim")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    return _dtype_code(q)


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, C: int = 64,
              phi: int = PHI_IDENTITY, decay_kind: int = DECAY_NONE, decay=None, state=None,
              out=None, workspace=None, stream=None, normalize: bool = False,
              norm_state=None, plan=None) -> torch.Tensor:
    """Chunkwise causal linear attention over [B,H,L,d] inputs; returns out [B,H,L,dv].

    `state` (fp32 [B,H,dk,dv]) is read as S_0 and overwritten with S_L when given.
    normalize: the normalised form (la_chunk_fwd_norm); `norm_state` (fp32
    [B,H,dk]) is read as z_0 and overwritten with z_L when given.
    plan: a launch-plan request (kernel, dv_tile, segments, groups, state_split), 0 =
    automatic (a shorter tuple leaves the remaining fields automatic);
    None takes the request of an enclosing `using_plan` block, if any.
    """
    dt = _qkv(q, k, v, 3)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    decay = _check_decay(decay, decay_kind, B, H, L, dk)
    _shape(state, "state", (B, H, dk, dv), torch.float32)
    _shape(norm_state, "norm_state", (B, H, dk), torch.float32)
    _shape(out, "out", (B, H, L, dv), q.dtype)
    if not normalize and norm_state is not None:
        raise ValueError("norm_state is for the normalised form (normalize=True)")
    request = _request(plan)
    if request is not None:
        need = _resolve(B, H, L, dk, dv, C, dt, decay_kind, normalize, request)[1]
    else:
        need = chunk_fwd_workspace_bytes(B, H, L, dk, dv, C, dt, decay_kind)
    _check_workspace(workspace, need)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (decay, "decay"), (state, "state"),
                 (out, "out"), (workspace, "workspace"), (norm_state, "norm_state")):
        _dev(t, n)
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=q.dtype, device=q.device)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    lib = load()
    if request is not None:
        _check(lib.la_chunk_fwd_planned(_ptr(q), _ptr(k), _ptr(v), dt, B, H, L, dk, dv, C, phi,
                                        decay_kind, _ptr(decay), _ptr(state), _ptr(norm_state),
                                        int(bool(normalize)), ctypes.byref(request), _ptr(out),
                                        _ptr(workspace), ws_bytes, _stream(stream)),
               "la_chunk_fwd_planned")
        return out
    if normalize:
        _check(lib.la_chunk_fwd_norm(_ptr(q), _ptr(k), _ptr(v), dt, B, H, L, dk, dv, C, phi,
                                     decay_kind, _ptr(decay), _ptr(state), _ptr(norm_state),
                                     _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)),
               "la_chunk_fwd_norm")
        return out
    _check(lib.la_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), dt, B, H, L, dk, dv, C, phi,
                            decay_kind, _ptr(decay), _ptr(state), _ptr(out), _ptr(workspace),
                            ws_bytes, _stream(stream)), "la_chunk_fwd")
    return out


def chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                      C: int = 64, phi: int = PHI_IDENTITY, decay_kind: int = DECAY_NONE,
                      decay=None, state=None, stream=None) -> torch.Tensor:
    """la_chunk_fwd_noalloc: the forward without a workspace, for callers that cannot
    allocate.  `out` ([B,H,L,dv], q's dtype) is required, since this call allocates
    nothing; the library's fixed per-device scratch stands in for the workspace."""
    dt = _qkv(q, k, v, 3)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    decay = _check_decay(decay, decay_kind, B, H, L, dk)
    _shape(state, "state", (B, H, dk, dv), torch.float32)
    if out is None:
        raise ValueError("chunk_fwd_noalloc needs out: it allocates nothing")
    _shape(out, "out", (B, H, L, dv), q.dtype)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (decay, "decay"), (state, "state"), (out, "out")):
        _dev(t, n)
    _check(load().la_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), dt, B, H, L, dk, dv, C, phi,
                                       decay_kind, _ptr(decay), _ptr(state), _ptr(out),
                                       _stream(stream)), "la_chunk_fwd_noalloc")
    return out


def _decode_decay(decay, decay_kind: int, N: int, H: int, dk: int, kinds=None):
    shape = {DECAY_NONE: None, DECAY_HEAD: (H,), DECAY_LOG: (N, H), DECAY_GATE: (N, H),
             DECAY_CHANNEL: (N, H, dk)}.get(decay_kind, "bad")
    if shape == "bad" or (kinds is not None and decay_kind not in kinds):
        raise ValueError(f"unsupported decay kind {decay_kind}")
    if shape is None:
        return None
    if decay is None:
        raise ValueError(f"decay kind {decay_kind} needs decay data of shape {shape}")
    _shape(decay, "decay", shape, torch.float32)
    return decay


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state: torch.Tensor,
                phi: int = PHI_IDENTITY, decay_kind: int = DECAY_NONE, decay=None, out=None,
                stream=None, norm_state=None) -> torch.Tensor:
    """One recurrent token for [N,H,d] inputs, updating `state` in place; returns o [N,H,dv].

    With `norm_state` (fp32 [N,H,dk], updated in place) the step is the
    normalised form (la_decode_step_norm).
    """
    if state is None:
        raise ValueError("decode_step needs the state")
    dt = _qkv(q, k, v, 2)
    N, H, dk = q.shape
    dv = v.shape[-1]
    decay = _decode_decay(decay, decay_kind, N, H, dk)
    _shape(state, "state", (N, H, dk, dv), torch.float32)
    _shape(norm_state, "norm_state", (N, H, dk), torch.float32)
    _shape(out, "out", (N, H, dv), q.dtype)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (state, "state"), (decay, "decay"), (out, "out"),
                 (norm_state, "norm_state")):
        _dev(t, n)
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    if norm_state is not None:
        _check(load().la_decode_step_norm(_ptr(q), _ptr(k), _ptr(v), dt, N, H, dk, dv, phi,
                                          decay_kind, _ptr(decay), _ptr(state), _ptr(norm_state),
                                          _ptr(out), _stream(stream)), "la_decode_step_norm")
        return out
    _check(load().la_decode_step(_ptr(q), _ptr(k), _ptr(v), dt, N, H, dk, dv, phi, decay_kind,
                                 _ptr(decay), _ptr(state), _ptr(out), _stream(stream)),
           "la_decode_step")
    return out


def delta_fwd_workspace_bytes(B: int, H: int, L: int, dk: int, dv: int, C: int,
                              dtype: int = LA_BF16) -> int:
    return int(load().la_delta_fwd_workspace_bytes(B, H, L, dk, dv, C, dtype))


def delta_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor, C: int = 64,
              decay_kind: int = DECAY_NONE, decay=None, state=None, out=None, workspace=None,
              stream=None) -> torch.Tensor:
    """The chunkwise delta rule (la_delta_fwd) over [B,H,L,d] inputs; beta fp32 [B,H,L].

    `state` (fp32 [B,H,dk,dv]) is read as S_0 and overwritten with S_L when given.
    """
    dt = _qkv(q, k, v, 3)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    if beta is None:
        raise ValueError("delta_fwd needs beta")
    _shape(beta, "beta", (B, H, L), torch.float32)
    decay = _check_decay(decay, decay_kind, B, H, L, dk,
                         kinds=(DECAY_NONE, DECAY_HEAD, DECAY_LOG, DECAY_GATE))
    _shape(state, "state", (B, H, dk, dv), torch.float32)
    _shape(out, "out", (B, H, L, dv), q.dtype)
    need = delta_fwd_workspace_bytes(B, H, L, dk, dv, C, dt)
    _check_workspace(workspace, need)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (beta, "beta"), (decay, "decay"),
                 (state, "state"), (out, "out"), (workspace, "workspace")):
        _dev(t, n)
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=q.dtype, device=q.device)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(load().la_delta_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), dt, B, H, L, dk, dv, C,
                               decay_kind, _ptr(decay), _ptr(state), _ptr(out), _ptr(workspace),
                               ws_bytes, _stream(stream)), "la_delta_fwd")
    return out


def delta_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                      state: torch.Tensor, decay_kind: int = DECAY_NONE, decay=None, out=None,
                      stream=None) -> torch.Tensor:
    """One delta-rule token for [N,H,d] inputs (beta fp32 [N,H]), updating `state` in place."""
    if state is None or beta is None:
        raise ValueError("delta_decode_step needs beta and the state")
    dt = _qkv(q, k, v, 2)
    N, H, dk = q.shape
    dv = v.shape[-1]
    _shape(beta, "beta", (N, H), torch.float32)
    decay = _decode_decay(decay, decay_kind, N, H, dk,
                          kinds=(DECAY_NONE, DECAY_HEAD, DECAY_LOG, DECAY_GATE))
    _shape(state, "state", (N, H, dk, dv), torch.float32)
    _shape(out, "out", (N, H, dv), q.dtype)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (beta, "beta"), (state, "state"),
                 (decay, "decay"), (out, "out")):
        _dev(t, n)
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    _check(load().la_delta_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), dt, N, H, dk, dv,
                                       decay_kind, _ptr(decay), _ptr(state), _ptr(out),
                                       _stream(stream)), "la_delta_decode_step")
    return out
