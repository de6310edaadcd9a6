"""ctypes binding over liblinattn.so (include/la.h).

Argument marshalling only: torch tensors supply device pointers, shapes and
the current HIP stream; every step of the computation runs in the library's
kernels.  There is no fallback: a missing library or a failed call raises.
"""
from __future__ import annotations

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
    """la_plan: kernel, value columns per workgroup, segments, column groups."""
    _fields_ = [("kernel", ctypes.c_int), ("dv_tile", ctypes.c_int),
                ("segments", ctypes.c_int), ("groups", ctypes.c_int)]

# every symbol include/la.h declares
EXPORTS = ("la_state_init", "la_chunk_fwd_workspace_bytes", "la_chunk_fwd", "la_decode_step",
           "la_status_string", "la_chunk_fwd_plan", "la_set_plan", "la_chunk_fwd_norm",
           "la_decode_step_norm", "la_delta_fwd_workspace_bytes", "la_delta_fwd",
           "la_delta_decode_step")

_lib = None


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
    lib.la_status_string.restype = ctypes.c_char_p
    lib.la_status_string.argtypes = [i]
    lib.la_chunk_fwd_plan.restype = i
    lib.la_chunk_fwd_plan.argtypes = [i] * 7 + [ctypes.POINTER(Plan)]
    lib.la_set_plan.restype = i
    lib.la_set_plan.argtypes = [ctypes.POINTER(Plan)]
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
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(status: int, where: str):
    if status != 0:
        raise LAError(status, where)


def plan(B: int, H: int, L: int, dk: int, dv: int, C: int, dtype: int = LA_BF16):
    """(kernel, value columns per workgroup, segments per head, column groups) of la_chunk_fwd."""
    p = Plan()
    _check(load().la_chunk_fwd_plan(B, H, L, dk, dv, C, dtype, ctypes.byref(p)),
           "la_chunk_fwd_plan")
    return p.kernel, p.dv_tile, p.segments, p.groups


def set_plan(kernel: int = 0, dv_tile: int = 0, segments: int = 0, groups: int = 0):
    """Override the bf16 launch plan process-wide (0 = automatic)."""
    p = Plan(int(kernel), int(dv_tile), int(segments), int(groups))
    _check(load().la_set_plan(ctypes.byref(p)), "la_set_plan")


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


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, C: int = 64,
              phi: int = PHI_IDENTITY, decay_kind: int = DECAY_NONE, decay=None, state=None,
              out=None, workspace=None, stream=None, normalize: bool = False,
              norm_state=None) -> torch.Tensor:
    """Chunkwise causal linear attention over [B,H,L,d] inputs; returns out [B,H,L,dv].

    `state` (fp32 [B,H,dk,dv]) is read as S_0 and overwritten with S_L when given.
    normalize: the normalised form (la_chunk_fwd_norm); `norm_state` (fp32
    [B,H,dk]) is read as z_0 and overwritten with z_L when given.
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (decay, "decay"), (state, "state"),
                 (out, "out"), (workspace, "workspace"), (norm_state, "norm_state")):
        _dev(t, n)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,H,L,dk] and v [B,H,L,dv]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=q.dtype, device=q.device)
    if decay is not None and decay.dtype != torch.float32:
        raise ValueError("decay data must be float32")
    if state is not None and (state.dtype != torch.float32 or tuple(state.shape) != (B, H, dk, dv)):
        raise ValueError("state must be float32 [B,H,dk,dv]")
    if norm_state is not None and (norm_state.dtype != torch.float32
                                   or tuple(norm_state.shape) != (B, H, dk)):
        raise ValueError("norm_state must be float32 [B,H,dk]")
    need = chunk_fwd_workspace_bytes(B, H, L, dk, dv, C, dt, decay_kind)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if normalize:
        _check(load().la_chunk_fwd_norm(_ptr(q), _ptr(k), _ptr(v), dt, B, H, L, dk, dv, C, phi,
                                        decay_kind, _ptr(decay), _ptr(state), _ptr(norm_state),
                                        _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)),
               "la_chunk_fwd_norm")
        return out
    _check(load().la_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), dt, B, H, L, dk, dv, C, phi,
                               decay_kind, _ptr(decay), _ptr(state), _ptr(out), _ptr(workspace),
                               ws_bytes, _stream(stream)), "la_chunk_fwd")
    return out


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state: torch.Tensor,
                phi: int = PHI_IDENTITY, decay_kind: int = DECAY_NONE, decay=None, out=None,
                stream=None, norm_state=None) -> torch.Tensor:
    """One recurrent token for [N,H,d] inputs, updating `state` in place; returns o [N,H,dv].

    With `norm_state` (fp32 [N,H,dk], updated in place) the step is the
    normalised form (la_decode_step_norm).
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (state, "state"), (decay, "decay"), (out, "out"),
                 (norm_state, "norm_state")):
        _dev(t, n)
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
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
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (beta, "beta"), (decay, "decay"),
                 (state, "state"), (out, "out"), (workspace, "workspace")):
        _dev(t, n)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,H,L,dk] and v [B,H,L,dv]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    if beta.dtype != torch.float32 or tuple(beta.shape) != (B, H, L):
        raise ValueError("beta must be float32 [B,H,L]")
    if decay is not None and decay.dtype != torch.float32:
        raise ValueError("decay data must be float32")
    if state is not None and (state.dtype != torch.float32 or tuple(state.shape) != (B, H, dk, dv)):
        raise ValueError("state must be float32 [B,H,dk,dv]")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=q.dtype, device=q.device)
    need = delta_fwd_workspace_bytes(B, H, L, dk, dv, C, dt)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().la_delta_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), dt, B, H, L, dk, dv, C,
                               decay_kind, _ptr(decay), _ptr(state), _ptr(out), _ptr(workspace),
                               ws_bytes, _stream(stream)), "la_delta_fwd")
    return out


def delta_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                      state: torch.Tensor, decay_kind: int = DECAY_NONE, decay=None, out=None,
                      stream=None) -> torch.Tensor:
    """One delta-rule token for [N,H,d] inputs (beta fp32 [N,H]), updating `state` in place."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (beta, "beta"), (state, "state"),
                 (decay, "decay"), (out, "out")):
        _dev(t, n)
    N, H, dk = q.shape
    dv = v.shape[-1]
    if beta.dtype != torch.float32 or tuple(beta.shape) != (N, H):
        raise ValueError("beta must be float32 [N,H]")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    _check(load().la_delta_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), dt, N, H, dk, dv,
                                       decay_kind, _ptr(decay), _ptr(state), _ptr(out),
                                       _stream(stream)), "la_delta_decode_step")
    return out

