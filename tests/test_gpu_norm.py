"""GPU parity of the normalised form (la_chunk_fwd_norm, la_decode_step_norm)
against the fp64 oracle: o_t = phi(q_t)^T S_t / phi(q_t)^T z_t with
z_t = a_t z_{t-1} + phi(k_t) (the linear/sparse attention tutorial, section
2.2).  phi = elu + 1 and a positive z_0 keep every denominator positive.
Bars as for the un-normalised form: 1e-4 (fp32), 1e-2 (bf16)."""
import numpy as np
import pytest
import torch

import oracle
from chunkwise_recurrence_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}
DEV = torch.device("cuda:0")


def _np(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def _z0(c: W.RandomCase):
    g = torch.Generator().manual_seed(c.seed + 7)
    return torch.rand((c.B, c.H, c.dk), generator=g) * 4.0 + 0.5


def _run(la, c: W.RandomCase, C: int, label: str):
    q, k, v, decay, S0 = W.random_inputs(c)
    S0 = S0 if S0 is not None else torch.zeros(c.B, c.H, c.dk, c.dv)
    z0 = _z0(c)
    print(f"[norm case] {label} B={c.B} H={c.H} L={c.L} dk={c.dk} dv={c.dv} C={C} "
          f"dtype={c.dtype} decay={c.decay_kind}", flush=True)
    S, z = S0.to(DEV).contiguous(), z0.to(DEV).contiguous()
    d = None if decay is None else decay.to(DEV).contiguous()
    out = la.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=C, phi=c.phi, decay_kind=c.decay_kind,
                       decay=d, state=S, normalize=True, norm_state=z)
    torch.cuda.synchronize()
    ref, ref_s, ref_z = oracle.recurrent(_np(q), _np(k), _np(v), c.phi, c.decay_kind, _np(decay),
                                         _np(S0), normalize=True, norm_state=_np(z0))
    tol = TOL[c.dtype]
    e = (oracle.rel_err(_np(out), ref), oracle.rel_err(_np(S), ref_s), oracle.rel_err(_np(z), ref_z))
    assert e[0] <= tol and e[1] <= tol and e[2] <= tol, f"{label}: out/state/z rel err {e}"
    return e


KINDS = [W.DECAY_NONE, W.DECAY_HEAD, W.DECAY_LOG, W.DECAY_GATE]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("d", [64, 128])
def test_norm_variants_bf16(gpu_lib, kind, d):
    c = W.RandomCase(2, 2, 64 * 5 + 23, d, d, torch.bfloat16, W.PHI_ELU1, kind, seed=300 + kind + d,
                     scale=1.0 / np.sqrt(d), gate_shift=-2.0, with_state=True)
    _run(gpu_lib, c, 64, "variants")


@pytest.mark.parametrize("kind", KINDS)
def test_norm_fp32(gpu_lib, kind):
    c = W.RandomCase(1, 2, 300, 16, 16, torch.float32, W.PHI_ELU1, kind, seed=320 + kind,
                     with_state=True)
    _run(gpu_lib, c, 64, "fp32 16")
    c = W.RandomCase(1, 2, 77, 32, 64, torch.float32, W.PHI_ELU1, kind, seed=330 + kind,
                     with_state=True)
    _run(gpu_lib, c, 32, "fp32 32x64")


@pytest.mark.parametrize("dk,dv,C", [(32, 32, 32), (64, 128, 64), (128, 64, 32), (128, 32, 64),
                                     (32, 128, 64), (64, 64, 128)])
def test_norm_head_dims(gpu_lib, dk, dv, C):
    c = W.RandomCase(1, 3, 200, dk, dv, torch.bfloat16, W.PHI_ELU1, W.DECAY_GATE,
                     seed=dk + dv + C, scale=1.0 / np.sqrt(dk), gate_shift=-2.0, with_state=True)
    _run(gpu_lib, c, C, "head dims")


@pytest.mark.parametrize("tile,segments,parts,split", [
    (128, 1, 2, 0), (128, 3, 2, 0), (128, 7, 1, 0), (64, 5, 2, 0), (32, 4, 2, 0), (128, 21, 2, 0),
    (64, 1, 2, 0), (32, 1, 1, 0), (128, 3, 2, 7), (64, 4, 2, 6), (128, 4, 1, 2)])
def test_norm_plan_invariance(gpu_lib, tile, segments, parts, split):
    la = gpu_lib
    with la.using_plan(la.KERNEL_STRIPE, tile, segments, parts, split):
        if split:
            assert la.plan(1, 2, 64 * 20 + 17, 128, 128, 64, normalize=True)[4] == split
        for kind in (W.DECAY_HEAD, W.DECAY_GATE, W.DECAY_NONE):
            c = W.RandomCase(1, 2, 64 * 20 + 17, 128, 128, torch.bfloat16, W.PHI_ELU1, kind,
                             seed=tile + segments + kind + split, scale=1.0 / np.sqrt(128),
                             gate_shift=-4.0, with_state=True)
            _run(la, c, 64, f"plan tile={tile} P={segments} parts={parts} split={split}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("kind", KINDS)
def test_norm_prefill_then_decode(gpu_lib, dtype, kind):
    la = gpu_lib
    L, n = 130, 5
    c = W.RandomCase(2, 2, L + n, 64, 64, dtype, W.PHI_ELU1, kind, seed=340 + kind,
                     scale=0.125, gate_shift=-2.0, with_state=True)
    q, k, v, d, S0 = W.random_inputs(c)
    z0 = _z0(c)
    S, z = S0.to(DEV).contiguous(), z0.to(DEV).contiguous()
    dd = None if d is None else d.to(DEV)
    pre = la.chunk_fwd(q[:, :, :L].contiguous().to(DEV), k[:, :, :L].contiguous().to(DEV),
                       v[:, :, :L].contiguous().to(DEV), C=32, phi=W.PHI_ELU1, decay_kind=kind,
                       decay=None if dd is None else (dd if kind == W.DECAY_HEAD
                                                      else dd[:, :, :L].contiguous()),
                       state=S, normalize=True, norm_state=z)
    steps = []
    for t in range(L, L + n):
        dstep = None if dd is None else (dd if kind == W.DECAY_HEAD else dd[:, :, t].contiguous())
        steps.append(la.decode_step(q[:, :, t].contiguous().to(DEV), k[:, :, t].contiguous().to(DEV),
                                    v[:, :, t].contiguous().to(DEV), S, phi=W.PHI_ELU1,
                                    decay_kind=kind, decay=dstep, norm_state=z))
    torch.cuda.synchronize()
    ref, ref_s, ref_z = oracle.recurrent(_np(q), _np(k), _np(v), W.PHI_ELU1, kind, _np(d),
                                         _np(S0), normalize=True, norm_state=_np(z0))
    tol = TOL[dtype]
    assert oracle.rel_err(_np(pre), ref[:, :, :L]) <= tol
    got = np.stack([_np(o) for o in steps], axis=2)
    assert oracle.rel_err(got, ref[:, :, L:]) <= tol
    assert oracle.rel_err(_np(S), ref_s) <= tol
    assert oracle.rel_err(_np(z), ref_z) <= tol


def test_norm_without_initial_z(gpu_lib):
    """norm_state = None: z_0 = 0, S_0 = 0; the first output equals v_0."""
    la = gpu_lib
    c = W.RandomCase(1, 2, 100, 64, 64, torch.bfloat16, W.PHI_ELU1, W.DECAY_HEAD, seed=360,
                     scale=0.125)
    q, k, v, d, _ = W.random_inputs(c)
    out = la.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=64, phi=W.PHI_ELU1,
                       decay_kind=W.DECAY_HEAD, decay=d.to(DEV), normalize=True)
    torch.cuda.synchronize()
    ref, _, _ = oracle.recurrent(_np(q), _np(k), _np(v), W.PHI_ELU1, W.DECAY_HEAD, _np(d),
                                 normalize=True)
    assert oracle.rel_err(_np(out), ref) <= 1e-2
    assert np.allclose(_np(out)[:, :, 0], _np(v)[:, :, 0], rtol=2e-2, atol=1e-3)


def test_norm_unsupported_shape_is_refused(gpu_lib):
    la = gpu_lib
    x = torch.zeros(1, 1, 64, 16, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(la.LAError):
        la.chunk_fwd(x, x, x, C=64, normalize=True)


def test_norm_on_the_full_retnet_shapes_whole_output(gpu_lib):
    """The normalised form at the size the benchmark times it: the retnet_bf16
    inputs ([2,32,16384,128], per-head gamma) with phi = elu+1, S_0 = 0 and
    z_0 = 0, in the automatic launch plan; every head against the oracle, the
    whole output, final state and final z compared."""
    la = gpu_lib
    w = W.WORKLOADS["retnet_bf16"]
    print(f"[norm case] full retnet shapes plan={la.plan(w.B, w.H, w.L, w.dk, w.dv, w.C, normalize=True)}",
          flush=True)
    q, k, v, gamma = W.chunk_inputs(w)
    S = torch.zeros(w.B, w.H, w.dk, w.dv, device=DEV)
    z = torch.zeros(w.B, w.H, w.dk, device=DEV)
    out = la.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=w.C, phi=W.PHI_ELU1,
                       decay_kind=w.decay_kind, decay=gamma.to(DEV), state=S, normalize=True,
                       norm_state=z)
    torch.cuda.synchronize()
    got_o, got_s, got_z = _np(out), _np(S), _np(z)
    del out, S, z
    ref_o, ref_s, ref_z = oracle.recurrent(_np(q), _np(k), _np(v), W.PHI_ELU1, W.DECAY_HEAD,
                                           _np(gamma), normalize=True)
    e = (oracle.rel_err(got_o, ref_o), oracle.rel_err(got_s, ref_s), oracle.rel_err(got_z, ref_z))
    print(f"normalised retnet shapes, all heads: out/state/z rel err {e}", flush=True)
    assert max(e) <= 1e-2, f"out/state/z rel err {e}"
