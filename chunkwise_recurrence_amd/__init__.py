"""Chunkwise causal linear attention on AMD MI355X (gfx950).

The compute lives in `liblinattn.so` (hand-written HIP kernels behind a C
ABI, declared in include/la.h).  This package is a thin ctypes binding over
it: every function marshals torch tensors into device pointers and a stream,
and the library does all of the work on the GPU.  There is no CPU fallback:
if the library cannot be loaded, calls raise.
"""
from .binding import (  # noqa: F401
    DECAY_CHANNEL, DECAY_GATE, DECAY_HEAD, DECAY_LOG, DECAY_NONE, PHI_ELU1, PHI_IDENTITY, LAError,
    EXPORTS, KERNEL_AUTO, KERNEL_F32, KERNEL_STRIP, KERNEL_STRIPE, LA_BF16, LA_F32, Plan,
    NOALLOC_SCRATCH_BYTES, chunk_fwd, chunk_fwd_noalloc, chunk_fwd_workspace_bytes, decode_step, delta_decode_step, delta_fwd,
    delta_fwd_workspace_bytes, lib_path, load, plan, plan_workspace_bytes, state_init, status_string,
    using_plan,
)
