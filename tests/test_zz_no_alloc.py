"""la_chunk_fwd_noalloc (the forward with the library's fixed per-device scratch
instead of a caller workspace) against la_chunk_fwd with a caller workspace,
both called through the C ABI: two calls in a row, the second on a smaller
problem, each must give bit-identical outputs and final states (same plan,
same kernels).  Both problems split their sequences into segments and use a
token decay, so the scratch holds segment states, the S_0 copy and the
in-chunk prefix sums."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from chunkwise_recurrence_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

# (B, H, L, d_k, d_v, phi, decay kind): the larger problem first
CASES = [(2, 8, 64 * 40 + 17, 128, 128, W.PHI_IDENTITY, W.DECAY_GATE),
         (1, 3, 64 * 9 + 5, 64, 64, W.PHI_ELU1, W.DECAY_LOG)]


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _run_pair(la, case, seed):
    B, H, L, dk, dv, phi, kind = case
    c = W.RandomCase(B, H, L, dk, dv, torch.bfloat16, phi, kind, seed=seed,
                     scale=1.0 / np.sqrt(dk), gate_shift=-4.0, with_state=True)
    q, k, v, decay, S0 = W.random_inputs(c)
    q, k, v, decay = q.to(DEV), k.to(DEV), v.to(DEV), decay.to(DEV)
    need = la.chunk_fwd_workspace_bytes(B, H, L, dk, dv, 64, la.LA_BF16, kind)
    assert 0 < need <= la.NOALLOC_SCRATCH_BYTES
    assert la.plan(B, H, L, dk, dv, 64)[2] > 1
    print(f"[no-alloc] case B={B} H={H} L={L} d={dk}x{dv} kind={kind} workspace={need}",
          flush=True)
    lib = la.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    S_ref, S_new = S0.to(DEV).contiguous(), S0.to(DEV).contiguous()
    out_ref, out_new = torch.empty_like(v), torch.full_like(v, float("nan"))
    st = lib.la_chunk_fwd(_p(q), _p(k), _p(v), la.LA_BF16, B, H, L, dk, dv, 64, phi, kind,
                          _p(decay), _p(S_ref), _p(out_ref), _p(ws), need, stream)
    assert st == 0, la.status_string(st)
    st = lib.la_chunk_fwd_noalloc(_p(q), _p(k), _p(v), la.LA_BF16, B, H, L, dk, dv, 64, phi,
                                  kind, _p(decay), _p(S_new), _p(out_new), stream)
    assert st == 0, la.status_string(st)
    torch.cuda.synchronize()
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    e_out, e_s = oracle.rel_err(f64(out_new), f64(out_ref)), oracle.rel_err(f64(S_new), f64(S_ref))
    print(f"[no-alloc] against la_chunk_fwd: out rel err {e_out:.2e}, state rel err {e_s:.2e}, "
          f"bit-identical {torch.equal(out_new, out_ref) and torch.equal(S_new, S_ref)}",
          flush=True)
    assert e_out <= 1e-2 and e_s <= 1e-2
    assert torch.equal(out_new, out_ref) and torch.equal(S_new, S_ref)


def test_noalloc_equals_the_workspace_forward_twice(gpu_lib):
    for i, case in enumerate(CASES):
        _run_pair(gpu_lib, case, seed=900 + i)


def test_noalloc_rejects_a_problem_beyond_its_scratch(gpu_lib):
    la = gpu_lib
    B, H, L, d = 1, 1, 1 << 24, 128
    assert la.chunk_fwd_workspace_bytes(B, H, L, d, d, 64, la.LA_BF16, W.DECAY_GATE) > \
        la.NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(1 << 20)  # never dereferenced: the size check comes first
    st = la.load().la_chunk_fwd_noalloc(p, p, p, la.LA_BF16, B, H, L, d, d, 64, 0, W.DECAY_GATE,
                                        p, None, p, None)
    assert st == 5  # LA_ERR_WORKSPACE
