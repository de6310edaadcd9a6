"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Error metric: max|out - ref| / max|ref| over the compared tensor (the pages'
"max relative difference").  Bars: 1e-4 for fp32 inputs, 1e-2 for bf16 inputs
with fp32 accumulation.  The oracle always receives the exact values the GPU
received (bf16 upcast to fp64).
"""
import numpy as np
import pytest
import torch

import oracle
from chunkwise_recurrence_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}


def _np(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def _gpu_fwd(la, q, k, v, C, phi, kind, decay, state):
    dev = torch.device("cuda:0")
    s = None if state is None else state.to(dev, torch.float32).contiguous()
    d = None if decay is None else decay.to(dev, torch.float32).contiguous()
    out = la.chunk_fwd(q.to(dev), k.to(dev), v.to(dev), C=C, phi=phi, decay_kind=kind, decay=d,
                       state=s)
    torch.cuda.synchronize()
    return out.cpu(), (None if s is None else s.cpu())


def _check_case(la, c: W.RandomCase, C: int, label: str = ""):
    q, k, v, decay, state = W.random_inputs(c)
    print(f"[case] {label} B={c.B} H={c.H} L={c.L} dk={c.dk} dv={c.dv} C={C} dtype={c.dtype} "
          f"phi={c.phi} decay={c.decay_kind} state={c.with_state}", flush=True)
    s_in = state if state is not None else torch.zeros(c.B, c.H, c.dk, c.dv)
    out, s_out = _gpu_fwd(la, q, k, v, C, c.phi, c.decay_kind, decay, s_in)
    ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), c.phi, c.decay_kind, _np(decay),
                                  _np(s_in))
    tol = TOL[c.dtype]
    e_out = oracle.rel_err(_np(out), ref)
    e_s = oracle.rel_err(_np(s_out), ref_s)
    assert e_out <= tol, f"{label} output rel err {e_out:.3e} > {tol}"
    assert e_s <= tol, f"{label} state rel err {e_s:.3e} > {tol}"
    return e_out, e_s


# --------------------------------------------------------------------------
# the 300 x 16 fp32 demo workload, whole
# --------------------------------------------------------------------------
def test_small_fp32_workload(gpu_lib):
    la = gpu_lib
    q, k, v = W.small_fp32_inputs()
    out, _ = _gpu_fwd(la, q, k, v, 64, la.PHI_IDENTITY, la.DECAY_NONE, None, None)
    ref, _ = oracle.recurrent(_np(q), _np(k), _np(v))
    err = oracle.rel_err(_np(out), ref)
    print(f"small_fp32 rel err {err:.3e}")
    assert err <= 1e-4


# --------------------------------------------------------------------------
# every variant, ragged lengths, several tiles, both dtypes
# --------------------------------------------------------------------------
VARIANTS = [(phi, kind) for phi in (0, 1) for kind in (0, 1, 2, 3)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("phi,kind", VARIANTS)
def test_variants_ragged(gpu_lib, dtype, phi, kind):
    sc = 1.0 / np.sqrt(64.0)
    for i, L in enumerate((1, 63, 65, 300)):
        c = W.RandomCase(2, 3, L, 64, 64, dtype, phi, kind, seed=100 + 10 * kind + phi + i,
                         scale=sc, with_state=True)
        _check_case(gpu_lib, c, 64, "variants")


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16),
                                   (16, 128), (64, 128)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_head_dims(gpu_lib, dk, dv, dtype):
    c = W.RandomCase(1, 2, 200, dk, dv, dtype, 0, W.DECAY_GATE, seed=7 + dk + dv,
                     scale=1.0 / np.sqrt(dk), gate_shift=-3.0, with_state=True)
    _check_case(gpu_lib, c, 64, "head_dims")


@pytest.mark.parametrize("C", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_chunk_sizes(gpu_lib, C, dtype):
    for L in (15, 127, 129, 515):
        c = W.RandomCase(1, 2, L, 128, 64, dtype, 1, W.DECAY_HEAD, seed=C + L,
                         scale=1.0 / np.sqrt(128), with_state=True)
        _check_case(gpu_lib, c, C, "chunk_sizes")


def test_chunk_size_invariance_on_gpu(gpu_lib):
    """Check [b] on the GPU: every C gives the same output up to bf16 rounding."""
    la = gpu_lib
    c = W.RandomCase(1, 4, 777, 64, 64, torch.bfloat16, 0, W.DECAY_GATE, seed=3, scale=0.125,
                     gate_shift=-4.0)
    q, k, v, d, _ = W.random_inputs(c)
    outs = [_np(_gpu_fwd(la, q, k, v, C, 0, W.DECAY_GATE, d, None)[0]) for C in (16, 32, 64, 128)]
    for o in outs[1:]:
        assert oracle.rel_err(o, outs[0]) < 1e-2


@pytest.mark.parametrize("kernel,tile,segments,groups", [
    (1, 16, 1, 1), (1, 32, 1, 1), (1, 64, 1, 1), (1, 32, 1, 2), (1, 64, 1, 2), (1, 32, 2, 1),
    (1, 32, 3, 2), (1, 64, 8, 1), (1, 64, 5, 2), (1, 64, 2, 2), (1, 16, 4, 1),
    (2, 128, 1, 1), (2, 64, 5, 1), (2, 32, 2, 1), (2, 128, 1, 2), (2, 64, 1, 2), (2, 32, 1, 2),
    (2, 128, 3, 2), (2, 64, 5, 2), (2, 32, 8, 2), (2, 128, 21, 2)])
def test_launch_plan_invariance(gpu_lib, kernel, tile, segments, groups):
    """Kernel, value tile, column groups and sequence segments change the work split,
    not the result."""
    la = gpu_lib
    with la.using_plan(kernel, tile, segments, groups):
        # 21 chunks: segments of ceil(21 / P) chunks, so P = 8 runs as 7 segments of 3
        got = la.plan(1, 2, 64 * 20 + 17, 128, 128, 64)
        assert got[:2] == (kernel, tile) and got[2] == -(-21 // -(-21 // segments))
        assert got[3] == groups
        for kind in (W.DECAY_NONE, W.DECAY_GATE, W.DECAY_HEAD):
            c = W.RandomCase(1, 2, 64 * 20 + 17, 128, 128, torch.bfloat16, 0, kind,
                             seed=tile + segments + kind, scale=1.0 / np.sqrt(128),
                             gate_shift=-5.0, with_state=True)
            _check_case(la, c, 64, f"plan kernel={kernel} tile={tile} P={segments} "
                                   f"groups={groups}")


@pytest.mark.parametrize("kernel,tile,segments,groups,split", [
    (1, 32, 2, 1, 4), (1, 64, 3, 2, 8), (1, 64, 4, 2, 3), (1, 16, 3, 1, 2), (2, 128, 3, 2, 4),
    (2, 64, 2, 1, 12), (2, 128, 5, 2, 5), (2, 128, 3, 2, 3)])
def test_state_split_invariance(gpu_lib, kernel, tile, segments, groups, split):
    """Splitting each segment's state pass over several workgroups (composed like
    segments) changes the work split, not the result."""
    la = gpu_lib
    L = 64 * 23 + 17  # 24 chunks, the last one ragged
    with la.using_plan(kernel, tile, segments, groups, split):
        got = la.plan(1, 2, L, 128, 128, 64)
        seg = -(-24 // segments)
        assert got[:4] == (kernel, tile, -(-24 // seg), groups)
        # a request is reduced to a divisor of the segment's chunk count
        want = max(s for s in range(1, split + 1) if seg % s == 0)
        assert got[4] == want and want > 1
        for kind in (W.DECAY_NONE, W.DECAY_GATE, W.DECAY_HEAD):
            c = W.RandomCase(1, 2, L, 128, 128, torch.bfloat16, 0, kind,
                             seed=600 + tile + segments + split + kind,
                             scale=1.0 / np.sqrt(128), gate_shift=-5.0, with_state=True)
            _check_case(la, c, 64, f"plan kernel={kernel} tile={tile} P={segments} "
                                   f"groups={groups} split={split}")


def test_resume_equals_one_call(gpu_lib):
    """chunk_fwd(L1) then chunk_fwd(L2) from its state == chunk_fwd(L1 + L2)."""
    la = gpu_lib
    c = W.RandomCase(2, 2, 700, 64, 64, torch.bfloat16, 1, W.DECAY_LOG, seed=21, scale=0.125)
    q, k, v, d, _ = W.random_inputs(c)
    dev = torch.device("cuda:0")
    qd, kd, vd, dd = q.to(dev), k.to(dev), v.to(dev), d.to(dev)
    S = torch.zeros(2, 2, 64, 64, device=dev)
    L1 = 333
    o1 = la.chunk_fwd(qd[:, :, :L1].contiguous(), kd[:, :, :L1].contiguous(),
                      vd[:, :, :L1].contiguous(), C=64, phi=1, decay_kind=W.DECAY_LOG,
                      decay=dd[:, :, :L1].contiguous(), state=S)
    o2 = la.chunk_fwd(qd[:, :, L1:].contiguous(), kd[:, :, L1:].contiguous(),
                      vd[:, :, L1:].contiguous(), C=64, phi=1, decay_kind=W.DECAY_LOG,
                      decay=dd[:, :, L1:].contiguous(), state=S)
    torch.cuda.synchronize()
    ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), 1, W.DECAY_LOG, _np(d))
    got = np.concatenate([_np(o1), _np(o2)], axis=2)
    assert oracle.rel_err(got, ref) < 1e-2
    assert oracle.rel_err(_np(S), ref_s) < 1e-2


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("phi,kind", VARIANTS)
def test_prefill_then_decode(gpu_lib, dtype, phi, kind):
    """chunk_fwd over L tokens, then n decode steps from its state == the recurrence over L + n."""
    la = gpu_lib
    L, n = 130, 6
    c = W.RandomCase(2, 3, L + n, 32, 64, dtype, phi, kind, seed=50 + kind + 5 * phi,
                     scale=1.0 / np.sqrt(32), with_state=True)
    q, k, v, d, S0 = W.random_inputs(c)
    dev = torch.device("cuda:0")
    S = S0.to(dev).contiguous()
    dd = None if d is None else d.to(dev)
    pre = la.chunk_fwd(q[:, :, :L].contiguous().to(dev), k[:, :, :L].contiguous().to(dev),
                       v[:, :, :L].contiguous().to(dev), C=32, phi=phi, decay_kind=kind,
                       decay=None if dd is None else (dd if kind == W.DECAY_HEAD
                                                      else dd[:, :, :L].contiguous()),
                       state=S)
    steps = []
    for t in range(L, L + n):
        dstep = None if dd is None else (dd if kind == W.DECAY_HEAD else dd[:, :, t].contiguous())
        steps.append(la.decode_step(q[:, :, t].contiguous().to(dev), k[:, :, t].contiguous().to(dev),
                                    v[:, :, t].contiguous().to(dev), S, phi=phi, decay_kind=kind,
                                    decay=dstep))
    torch.cuda.synchronize()
    ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), phi, kind, _np(d), _np(S0))
    tol = TOL[dtype]
    assert oracle.rel_err(_np(pre), ref[:, :, :L]) <= tol
    got = np.stack([_np(o) for o in steps], axis=2)
    assert oracle.rel_err(got, ref[:, :, L:]) <= tol
    assert oracle.rel_err(_np(S), ref_s) <= tol


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (128, 32), (64, 64), (128, 128)])
def test_decode_head_dims(gpu_lib, dk, dv):
    la = gpu_lib
    N, H, T = 5, 3, 4
    g = torch.Generator().manual_seed(dk * 1000 + dv)
    S0 = torch.randn(N, H, dk, dv, generator=g) * 0.1
    dev = torch.device("cuda:0")
    S = S0.to(dev)
    ref_S = _np(S0)
    for t in range(T):
        q, k, v = (torch.randn(N, H, d, generator=g).to(torch.bfloat16) for d in (dk, dk, dv))
        gate = torch.randn(N, H, generator=g)
        o = la.decode_step(q.to(dev), k.to(dev), v.to(dev), S, phi=0, decay_kind=W.DECAY_GATE,
                           decay=gate.to(dev))
        torch.cuda.synchronize()
        ro, ref_S = oracle.decode_step(_np(q), _np(k), _np(v), 0, W.DECAY_GATE, _np(gate), ref_S)
        assert oracle.rel_err(_np(o), ro) < 1e-2
    assert oracle.rel_err(_np(S), ref_S) < 1e-5  # the state itself stays fp32


def test_zero_length_is_a_noop(gpu_lib):
    la = gpu_lib
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device=dev)
    S = torch.randn(1, 2, 64, 64, device=dev)
    S_before = S.clone()
    out = la.chunk_fwd(q, q, q, C=64, state=S)
    torch.cuda.synchronize()
    assert out.shape == (1, 2, 0, 64) and torch.equal(S, S_before)


def test_state_init_zeroes(gpu_lib):
    la = gpu_lib
    S = torch.randn(3, 5, 32, 64, device="cuda:0")
    la.state_init(S)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S).item() == 0


def test_head_permutation_equivariance(gpu_lib):
    """Heads are independent: permuting them permutes the outputs (bit-exact)."""
    la = gpu_lib
    c = W.RandomCase(1, 6, 333, 64, 64, torch.bfloat16, 1, W.DECAY_NONE, seed=77, scale=0.125)
    q, k, v, _, _ = W.random_inputs(c)
    perm = torch.tensor([3, 0, 5, 1, 4, 2])
    o, _ = _gpu_fwd(la, q, k, v, 64, 1, 0, None, None)
    op, _ = _gpu_fwd(la, q[:, perm].contiguous(), k[:, perm].contiguous(), v[:, perm].contiguous(),
                     64, 1, 0, None, None)
    assert torch.equal(o[:, perm], op)


# --------------------------------------------------------------------------
# degenerate decays: a = 1, a -> 0, gates saturated both ways
# --------------------------------------------------------------------------
def _degenerate_inputs(dk, dv, H, L, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(1, H, L, dk, generator=g) / np.sqrt(dk)).to(dtype)
    k = (torch.randn(1, H, L, dk, generator=g) / np.sqrt(dk)).to(dtype)
    v = torch.randn(1, H, L, dv, generator=g).to(dtype)
    s0 = torch.randn(1, H, dk, dv, generator=g) * 0.1
    # per token, saturated gates: g = +30 (a = e^-30, nearly a reset) or g = -30
    # (a = 1 to fp32 precision), and ordinary ones, mixed at random
    pick = torch.randint(0, 3, (1, H, L), generator=g)
    gate = torch.where(pick == 0, torch.full((1, H, L), 30.0),
                       torch.where(pick == 1, torch.full((1, H, L), -30.0),
                                   torch.randn(1, H, L, generator=g)))
    return q, k, v, s0, gate


@pytest.mark.parametrize("dtype,dk,dv,plan", [
    (torch.bfloat16, 128, 128, (0, 0, 0, 0)), (torch.bfloat16, 128, 128, (2, 128, 3, 2)),
    (torch.bfloat16, 64, 64, (0, 0, 0, 0)), (torch.bfloat16, 64, 64, (1, 32, 4, 1)),
    (torch.float32, 32, 64, (0, 0, 0, 0))])
def test_degenerate_decays(gpu_lib, dtype, dk, dv, plan):
    """gamma = 1 exactly, gamma = 1e-20 (the a -> 0 limit: every step forgets the
    past), 1 - 2^-20 and 0.5 across heads; saturated gates both ways per token.
    Exponents reach -4e3 in log2 units: no inf - inf, no NaN, and a carried
    state of fp32 zeros where the decay wipes it."""
    la = gpu_lib
    with la.using_plan(*plan):
        H, L = 4, 64 * 6 + 29
        q, k, v, s0, gate = _degenerate_inputs(dk, dv, H, L, dtype, seed=dk + dv + plan[2])
        gamma = torch.tensor([1.0, 1e-20, 1.0 - 2.0 ** -20, 0.5], dtype=torch.float32)
        tol = TOL[dtype]
        for kind, d in ((W.DECAY_HEAD, gamma), (W.DECAY_GATE, gate)):
            out, s_out = _gpu_fwd(la, q, k, v, 64, 0, kind, d, s0)
            ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), 0, kind, _np(d), _np(s0))
            assert torch.isfinite(out.float()).all() and torch.isfinite(s_out).all()
            e_out, e_s = oracle.rel_err(_np(out), ref), oracle.rel_err(_np(s_out), ref_s)
            print(f"[degenerate] plan={plan} dtype={dtype} kind={kind}: out {e_out:.2e} "
                  f"state {e_s:.2e}", flush=True)
            assert e_out <= tol and e_s <= tol
            if kind == W.DECAY_HEAD:
                # head 1 (gamma = 1e-20) keeps only the current token:
                # o_t = (q_t . k_t) v_t, a closed form independent of the oracle
                qd, kd, vd = (_np(x[0, 1]) for x in (q, k, v))
                closed = (qd * kd).sum(-1, keepdims=True) * vd
                got = _np(out[0, 1])
                assert np.abs(got - closed).max() <= tol * np.abs(closed).max()


def test_decode_degenerate_decays(gpu_lib):
    """Decode steps with gamma = 1, 1e-20 (S' = k v^T: the step forgets the
    state), 1 - 2^-20 and 0.5 across heads, then with saturated gates."""
    la = gpu_lib
    dev = torch.device("cuda:0")
    N, H, d = 4, 4, 128
    g = torch.Generator().manual_seed(990)
    S0 = torch.randn(N, H, d, d, generator=g) * 0.1
    gamma = torch.tensor([1.0, 1e-20, 1.0 - 2.0 ** -20, 0.5], dtype=torch.float32)
    for kind in (W.DECAY_HEAD, W.DECAY_GATE):
        S = S0.to(dev).contiguous()
        ref_S = _np(S0)
        for t in range(3):
            q, k, v = ((torch.randn(N, H, d, generator=g) / np.sqrt(d)).to(torch.bfloat16)
                       for _ in range(3))
            if kind == W.DECAY_HEAD:
                dd = gamma
            else:
                dd = torch.where(torch.rand(N, H, generator=g) < 0.5, torch.full((N, H), 30.0),
                                 torch.full((N, H), -30.0))
            o = la.decode_step(q.to(dev), k.to(dev), v.to(dev), S, decay_kind=kind,
                               decay=dd.to(dev))
            torch.cuda.synchronize()
            ro, ref_S = oracle.decode_step(_np(q), _np(k), _np(v), 0, kind, _np(dd), ref_S)
            assert torch.isfinite(o.float()).all()
            assert oracle.rel_err(_np(o), ro) < 1e-2
        assert oracle.rel_err(_np(S), ref_S) < 1e-5
        if kind == W.DECAY_HEAD:
            # head 1 keeps only the last token's k v^T
            kd, vd = _np(k[:, 1]), _np(v[:, 1])
            outer = kd[:, :, None] * vd[:, None, :]
            assert np.abs(_np(S[:, 1]) - outer).max() <= 1e-5 * np.abs(outer).max()
