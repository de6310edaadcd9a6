"""GPU parity of the per-channel gate (LA_DECAY_CHANNEL_LOG, GLA's diagonal
decay, the linear/sparse attention tutorial's section 2.4):
S_t = diag(a_t) S_{t-1} + phi(k_t) v_t^T with log a_t in [B,H,L,d_k], against
the fp64 token-by-token oracle.  Bars as for the other decays: 1e-4 (fp32),
1e-2 (bf16 inputs), as max|err| / max|ref|."""
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


def _run(la, c: W.RandomCase, C: int, label: str):
    q, k, v, decay, S0 = W.random_inputs(c)
    S0 = S0 if S0 is not None else torch.zeros(c.B, c.H, c.dk, c.dv)
    print(f"[channel case] {label} B={c.B} H={c.H} L={c.L} dk={c.dk} dv={c.dv} C={C} "
          f"dtype={c.dtype} phi={c.phi} mean={c.channel_mean}", flush=True)
    S = S0.to(DEV).contiguous()
    out = la.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=C, phi=c.phi,
                       decay_kind=W.DECAY_CHANNEL, decay=decay.to(DEV).contiguous(), state=S)
    torch.cuda.synchronize()
    ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), c.phi, W.DECAY_CHANNEL, _np(decay),
                                  _np(S0))
    tol = TOL[c.dtype]
    e = (oracle.rel_err(_np(out), ref), oracle.rel_err(_np(S), ref_s))
    assert e[0] <= tol and e[1] <= tol, f"{label}: out/state rel err {e}"
    return e


@pytest.mark.parametrize("mean", [0.05, 1.0])
@pytest.mark.parametrize("phi", [W.PHI_IDENTITY, W.PHI_ELU1])
@pytest.mark.parametrize("d", [64, 128])
def test_channel_variants_bf16(gpu_lib, d, phi, mean):
    """Ragged length (5 chunks of 64 and 23 tokens), an initial state, weak and strong decay."""
    c = W.RandomCase(2, 2, 64 * 5 + 23, d, d, torch.bfloat16, phi, W.DECAY_CHANNEL,
                     seed=400 + d + 10 * phi + int(100 * mean), scale=1.0 / np.sqrt(d),
                     channel_mean=mean, with_state=True)
    _run(gpu_lib, c, 64, "variants")


@pytest.mark.parametrize("phi", [W.PHI_IDENTITY, W.PHI_ELU1])
def test_channel_fp32(gpu_lib, phi):
    c = W.RandomCase(1, 2, 300, 16, 16, torch.float32, phi, W.DECAY_CHANNEL, seed=430 + phi,
                     channel_mean=0.3, with_state=True)
    _run(gpu_lib, c, 64, "fp32 16")
    c = W.RandomCase(1, 2, 77, 32, 64, torch.float32, phi, W.DECAY_CHANNEL, seed=440 + phi,
                     channel_mean=0.3, with_state=True)
    _run(gpu_lib, c, 32, "fp32 32x64")


@pytest.mark.parametrize("dk,dv,C", [(32, 32, 32), (64, 128, 64), (128, 64, 32), (32, 128, 128),
                                     (32, 64, 128), (64, 32, 64), (128, 32, 32), (128, 128, 32)])
def test_channel_head_dims(gpu_lib, dk, dv, C):
    # the mean keeps every chunk's summed log decay within the split's range
    c = W.RandomCase(1, 3, 200, dk, dv, torch.bfloat16, W.PHI_IDENTITY, W.DECAY_CHANNEL,
                     seed=dk + dv + C + 7, scale=1.0 / np.sqrt(dk), channel_mean=0.4,
                     with_state=True)
    _run(gpu_lib, c, C, "head dims")


@pytest.mark.parametrize("tile,segments,parts,split", [
    (128, 1, 2, 0), (128, 3, 2, 0), (128, 7, 1, 0), (64, 5, 2, 0), (64, 2, 2, 0), (128, 21, 2, 0),
    (128, 3, 2, 4), (64, 7, 2, 2), (128, 3, 1, 8)])
def test_channel_plan_invariance(gpu_lib, tile, segments, parts, split):
    """Value tiles, key parts, sequence segments and state-pass splits (the scans
    compose per-channel decays) all give the oracle's result."""
    la = gpu_lib
    with la.using_plan(la.KERNEL_STRIPE, tile, segments, parts, split):
        if split:
            assert la.plan(1, 2, 64 * 21 + 5, 128, 128, 64, decay_kind=4)[4] == split
        c = W.RandomCase(1, 2, 64 * 21 + 5, 128, 128, torch.bfloat16, W.PHI_IDENTITY,
                         W.DECAY_CHANNEL, seed=460 + tile + segments + parts + split,
                         scale=1.0 / np.sqrt(128), channel_mean=0.02, with_state=True)
        _run(la, c, 64, f"plan tile={tile} P={segments} parts={parts} split={split}")


def test_channel_broadcast_equals_token_decay(gpu_lib):
    """log a[t, d] = log a[t] for every channel is the per-token decay: both
    kinds agree with each other and with the oracle."""
    la = gpu_lib
    c = W.RandomCase(1, 2, 64 * 4 + 9, 128, 128, torch.bfloat16, W.PHI_IDENTITY, W.DECAY_LOG,
                     seed=470, scale=1.0 / np.sqrt(128), with_state=True)
    q, k, v, log_a, S0 = W.random_inputs(c)
    chan = log_a[..., None].expand(c.B, c.H, c.L, c.dk).contiguous()
    S1, S2 = S0.to(DEV).contiguous(), S0.to(DEV).contiguous()
    o1 = la.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=64, decay_kind=W.DECAY_LOG,
                      decay=log_a.to(DEV), state=S1)
    o2 = la.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=64, decay_kind=W.DECAY_CHANNEL,
                      decay=chan.to(DEV), state=S2)
    torch.cuda.synchronize()
    ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), 0, W.DECAY_LOG, _np(log_a), _np(S0))
    assert oracle.rel_err(_np(o2), ref) <= 1e-2 and oracle.rel_err(_np(S2), ref_s) <= 1e-2
    assert oracle.rel_err(_np(o2), _np(o1)) <= 1e-2
    assert oracle.rel_err(_np(S2), _np(S1)) <= 1e-2


def test_channel_zero_decay_is_ungated(gpu_lib):
    """log a = 0 (a = 1) reduces to the ungated form."""
    la = gpu_lib
    c = W.RandomCase(2, 2, 150, 64, 64, torch.bfloat16, W.PHI_ELU1, W.DECAY_NONE, seed=480,
                     scale=1.0 / np.sqrt(64), with_state=True)
    q, k, v, _, S0 = W.random_inputs(c)
    S = S0.to(DEV).contiguous()
    out = la.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=64, phi=W.PHI_ELU1,
                       decay_kind=W.DECAY_CHANNEL, decay=torch.zeros(2, 2, 150, 64, device=DEV),
                       state=S)
    torch.cuda.synchronize()
    ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), W.PHI_ELU1, W.DECAY_NONE, None, _np(S0))
    assert oracle.rel_err(_np(out), ref) <= 1e-2 and oracle.rel_err(_np(S), ref_s) <= 1e-2


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_channel_prefill_then_decode(gpu_lib, dtype):
    """chunk_fwd over L tokens, then n decode steps from its state == the recurrence over L + n."""
    la = gpu_lib
    L, n = 130, 6
    c = W.RandomCase(2, 3, L + n, 64, 64, dtype, W.PHI_IDENTITY, W.DECAY_CHANNEL, seed=490,
                     scale=1.0 / np.sqrt(64), channel_mean=0.2, with_state=True)
    q, k, v, d, S0 = W.random_inputs(c)
    S = S0.to(DEV).contiguous()
    dd = d.to(DEV)
    pre = la.chunk_fwd(q[:, :, :L].contiguous().to(DEV), k[:, :, :L].contiguous().to(DEV),
                       v[:, :, :L].contiguous().to(DEV), C=32, decay_kind=W.DECAY_CHANNEL,
                       decay=dd[:, :, :L].contiguous(), state=S)
    steps = []
    for t in range(L, L + n):
        steps.append(la.decode_step(q[:, :, t].contiguous().to(DEV), k[:, :, t].contiguous().to(DEV),
                                    v[:, :, t].contiguous().to(DEV), S, decay_kind=W.DECAY_CHANNEL,
                                    decay=dd[:, :, t].contiguous()))
    torch.cuda.synchronize()
    ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), 0, W.DECAY_CHANNEL, _np(d), _np(S0))
    tol = TOL[dtype]
    assert oracle.rel_err(_np(pre), ref[:, :, :L]) <= tol
    got = np.stack([_np(o) for o in steps], axis=2)
    assert oracle.rel_err(got, ref[:, :, L:]) <= tol
    assert oracle.rel_err(_np(S), ref_s) <= tol


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (128, 32), (128, 128)])
def test_channel_decode_head_dims(gpu_lib, dk, dv):
    la = gpu_lib
    N, H, T = 5, 3, 4
    g = torch.Generator().manual_seed(dk * 1000 + dv + 1)
    S0 = torch.randn(N, H, dk, dv, generator=g) * 0.1
    S = S0.to(DEV)
    ref_S = _np(S0)
    for _ in range(T):
        q, k, v = (torch.randn(N, H, d, generator=g).to(torch.bfloat16) for d in (dk, dk, dv))
        log_a = -torch.rand(N, H, dk, generator=g)
        o = la.decode_step(q.to(DEV), k.to(DEV), v.to(DEV), S, decay_kind=W.DECAY_CHANNEL,
                           decay=log_a.to(DEV))
        torch.cuda.synchronize()
        ro, ref_S = oracle.decode_step(_np(q), _np(k), _np(v), 0, W.DECAY_CHANNEL, _np(log_a),
                                       ref_S)
        assert oracle.rel_err(_np(o), ro) < 1e-2
    assert oracle.rel_err(_np(S), ref_S) < 1e-5  # the state itself stays fp32


def test_gla_workload_whole_output(gpu_lib):
    """The full gla_bf16 workload (B=2, H=32, L=16384, d=128, C=64) in the
    bench's launch configuration; the oracle recomputes every head, and the
    whole output and final state are compared."""
    la = gpu_lib
    w = W.WORKLOADS["gla_bf16"]
    print(f"[workload] gla_bf16 plan={la.plan(w.B, w.H, w.L, w.dk, w.dv, w.C, decay_kind=4)}",
          flush=True)
    q, k, v, decay = W.chunk_inputs(w)
    S = torch.zeros(w.B, w.H, w.dk, w.dv, device=DEV)
    out = la.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=w.C, decay_kind=W.DECAY_CHANNEL,
                       decay=decay.to(DEV), state=S)
    torch.cuda.synchronize()
    got, got_s = _np(out), _np(S)
    del out, S
    ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), 0, W.DECAY_CHANNEL, _np(decay))
    e_out, e_s = oracle.rel_err(got, ref), oracle.rel_err(got_s, ref_s)
    print(f"gla_bf16: all heads: output rel err {e_out:.3e}, state rel err {e_s:.3e}", flush=True)
    assert e_out <= 1e-2 and e_s <= 1e-2


@pytest.mark.parametrize("phi", [W.PHI_IDENTITY, W.PHI_ELU1])
def test_channel_normalised_fp32(gpu_lib, phi):
    """fp32 inputs take the normalised form with the per-channel gate:
    z_t = diag(a_t) z_{t-1} + phi(k_t), o_t = phi(q_t)^T S_t / phi(q_t)^T z_t."""
    la = gpu_lib
    c = W.RandomCase(1, 2, 150, 32, 64, torch.float32, phi, W.DECAY_CHANNEL, seed=500 + phi,
                     channel_mean=0.2, with_state=True)
    q, k, v, decay, S0 = W.random_inputs(c)
    if phi == W.PHI_IDENTITY:  # keep every denominator away from zero
        q, k = q.abs() + 0.1, k.abs() + 0.1
    g = torch.Generator().manual_seed(501)
    z0 = torch.rand((1, 2, 32), generator=g) * 4.0 + 0.5
    S, z = S0.to(DEV).contiguous(), z0.to(DEV).contiguous()
    out = la.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=32, phi=phi, decay_kind=W.DECAY_CHANNEL,
                       decay=decay.to(DEV), state=S, normalize=True, norm_state=z)
    torch.cuda.synchronize()
    ref, ref_s, ref_z = oracle.recurrent(_np(q), _np(k), _np(v), phi, W.DECAY_CHANNEL, _np(decay),
                                         _np(S0), normalize=True, norm_state=_np(z0))
    assert oracle.rel_err(_np(out), ref) <= 1e-4
    assert oracle.rel_err(_np(S), ref_s) <= 1e-4 and oracle.rel_err(_np(z), ref_z) <= 1e-4
    # and the decode step continues it
    Sd, zd = S.clone(), z.clone()
    qd, kd, vd = (x[:, :, 0].contiguous() for x in (q, k, v))
    ld = decay[:, :, 0].contiguous()
    od = la.decode_step(qd.to(DEV), kd.to(DEV), vd.to(DEV), Sd, phi=phi,
                        decay_kind=W.DECAY_CHANNEL, decay=ld.to(DEV), norm_state=zd)
    torch.cuda.synchronize()
    ro, rs, rz = oracle.decode_step(_np(qd), _np(kd), _np(vd), phi, W.DECAY_CHANNEL, _np(ld),
                                    ref_s, normalize=True, norm_state=ref_z)
    assert oracle.rel_err(_np(od), ro) <= 1e-4 and oracle.rel_err(_np(zd), rz) <= 1e-4


def _strong_log_decay(pattern, B, H, L, dk, seed):
    """Per-channel log decays far past the split's range (a chunk's log2 decay
    summing below -192 in some channel), for the exact re-run."""
    g = torch.Generator().manual_seed(seed)
    mild = -torch.empty((B, H, L, dk)).exponential_(1.0 / 0.05, generator=g)
    if pattern == "uniform_2.2":       # every chunk: 64 x -2.2 = -140.8 (-203 in log2)
        return torch.full((B, H, L, dk), -2.2)
    if pattern == "uniform_16":        # every chunk sums to about -1e3
        return torch.full((B, H, L, dk), -16.0)
    if pattern == "forget_all":        # a = 0 everywhere: S_t = k_t v_t^T
        return torch.full((B, H, L, dk), -float("inf"))
    if pattern == "mixed":
        # mild decays, with some channels of some chunks forgetting (-inf) or
        # decaying by e^-1000 at single tokens, and whole strong chunks in one head
        x = mild.clone()
        sel = torch.rand((B, H, L, dk), generator=g)
        x[sel < 0.004] = -float("inf")
        x[(sel >= 0.004) & (sel < 0.008)] = -1000.0
        x[:, -1, 64:128] = -3.0
        return x
    if pattern == "alternating":       # strong and mild chunks in turn
        x = mild.clone()
        for c0 in range(0, L, 128):
            x[..., c0:c0 + 64, :] = -4.0
        return x
    raise ValueError(pattern)


@pytest.mark.parametrize("pattern", ["uniform_2.2", "uniform_16", "forget_all", "mixed",
                                     "alternating"])
@pytest.mark.parametrize("plan", [(0, 0, 0, 0), (2, 128, 1, 2), (2, 128, 3, 2), (2, 64, 2, 2)])
def test_channel_strong_decay_exact(gpu_lib, pattern, plan):
    """bf16 per-channel gate at decays of any strength: chunks whose log2 decay
    sums below -192 in some channel are recomputed by the exact pass (scores
    per element with direct-sum exponents), the others keep the split; every
    plan (one segment: the re-run reads a copy of S_0; several: the state
    pass's exact update and the selected composition) gives the oracle's
    result, and no inf or NaN appears."""
    la = gpu_lib
    B, H, L, d = 1, 3, 64 * 7 + 21, 128
    c = W.RandomCase(B, H, L, d, d, torch.bfloat16, W.PHI_ELU1 if pattern == "mixed" else 0,
                     W.DECAY_CHANNEL, seed=530 + len(pattern) + plan[2],
                     scale=1.0 / np.sqrt(d), with_state=True)
    q, k, v, _, S0 = W.random_inputs(c)
    decay = _strong_log_decay(pattern, B, H, L, d, seed=531)
    print(f"[channel strong] pattern={pattern} plan={plan}", flush=True)
    with la.using_plan(*plan):
        S = S0.to(DEV).contiguous()
        out = la.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=64, phi=c.phi,
                           decay_kind=W.DECAY_CHANNEL, decay=decay.to(DEV), state=S)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(S).all()
    ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), c.phi, W.DECAY_CHANNEL, _np(decay),
                                  _np(S0))
    e = (oracle.rel_err(_np(out), ref), oracle.rel_err(_np(S), ref_s))
    print(f"[channel strong] pattern={pattern} plan={plan}: out/state rel err {e}", flush=True)
    assert e[0] <= 1e-2 and e[1] <= 1e-2
    if pattern == "forget_all":
        # a closed form that needs no oracle: o_t = (phi(q_t) . phi(k_t)) v_t, S_L = k_L v_L^T
        qd, kd, vd = _np(q), _np(k), _np(v)
        closed = (qd * kd).sum(-1, keepdims=True) * vd
        assert np.abs(_np(out) - closed).max() <= 1e-2 * np.abs(closed).max()
        last = kd[:, :, -1, :, None] * vd[:, :, -1, None, :]
        assert np.abs(_np(S) - last).max() <= 1e-2 * np.abs(last).max()


@pytest.mark.parametrize("dk,dv,C", [(64, 64, 64), (128, 32, 32), (32, 128, 128), (64, 32, 64)])
def test_channel_strong_decay_exact_head_dims(gpu_lib, dk, dv, C):
    """The exact pass on the other layouts the per-channel gate takes."""
    la = gpu_lib
    B, H, L = 1, 2, 3 * C + 9
    c = W.RandomCase(B, H, L, dk, dv, torch.bfloat16, W.PHI_IDENTITY, W.DECAY_CHANNEL,
                     seed=560 + dk + dv + C, scale=1.0 / np.sqrt(dk), with_state=True)
    q, k, v, _, S0 = W.random_inputs(c)
    decay = _strong_log_decay("mixed", B, H, L, dk, seed=561)
    decay[:, 0, C:2 * C] = -9.0
    S = S0.to(DEV).contiguous()
    out = la.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=C, decay_kind=W.DECAY_CHANNEL,
                       decay=decay.to(DEV), state=S)
    torch.cuda.synchronize()
    ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), 0, W.DECAY_CHANNEL, _np(decay), _np(S0))
    e = (oracle.rel_err(_np(out), ref), oracle.rel_err(_np(S), ref_s))
    print(f"[channel strong] dk={dk} dv={dv} C={C}: out/state rel err {e}", flush=True)
    assert e[0] <= 1e-2 and e[1] <= 1e-2


def test_channel_strong_decay_fp32_and_decode(gpu_lib):
    """fp32 inputs and the decode step with forgetting channels (log a = -inf) and
    e^-1000 steps: no NaN, the oracle's result (fp32 bar)."""
    la = gpu_lib
    B, H, L, d = 1, 2, 150, 32
    c = W.RandomCase(B, H, L, d, d, torch.float32, W.PHI_IDENTITY, W.DECAY_CHANNEL, seed=570,
                     with_state=True)
    q, k, v, _, S0 = W.random_inputs(c)
    decay = _strong_log_decay("mixed", B, H, L, d, seed=571)
    S = S0.to(DEV).contiguous()
    out = la.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=64, decay_kind=W.DECAY_CHANNEL,
                       decay=decay.to(DEV), state=S)
    torch.cuda.synchronize()
    ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), 0, W.DECAY_CHANNEL, _np(decay), _np(S0))
    e = (oracle.rel_err(_np(out), ref), oracle.rel_err(_np(S), ref_s))
    print(f"[channel strong] fp32: out/state rel err {e}", flush=True)
    assert e[0] <= 1e-4 and e[1] <= 1e-4
    # decode: three steps, the first forgetting every channel of head 0
    Sd = S0.to(DEV).contiguous()
    ref_S = _np(S0)
    for t in range(3):
        ld = decay[:, :, t].clone()
        if t == 0:
            ld[:, 0] = -float("inf")
        o = la.decode_step(q[:, :, t].contiguous().to(DEV), k[:, :, t].contiguous().to(DEV),
                           v[:, :, t].contiguous().to(DEV), Sd, decay_kind=W.DECAY_CHANNEL,
                           decay=ld.to(DEV))
        torch.cuda.synchronize()
        ro, ref_S = oracle.decode_step(_np(q[:, :, t]), _np(k[:, :, t]), _np(v[:, :, t]), 0,
                                       W.DECAY_CHANNEL, _np(ld), ref_S)
        assert oracle.rel_err(_np(o), ro) <= 1e-4
    assert oracle.rel_err(_np(Sd), ref_S) <= 1e-5


# (d_k, value tile, key parts, C): every layout of the per-channel prefix scan
# -- a wave's d_k / waves channels in groups of 4 (or 2) lanes' channels times
# R runs of a 16-lane row, R = 2 .. 16 -- and both forms of the output pass
@pytest.mark.parametrize("dk,tile,parts,C", [
    (128, 128, 2, 64), (128, 128, 1, 64), (128, 64, 2, 64), (128, 64, 1, 32), (128, 32, 2, 32),
    (64, 128, 2, 64), (64, 128, 1, 32), (64, 64, 1, 64), (64, 32, 2, 64),
    (32, 32, 1, 64), (32, 64, 1, 32), (32, 128, 1, 64), (32, 128, 1, 128)])
@pytest.mark.parametrize("strength", ["mild", "strong"])
def test_channel_scan_layouts(gpu_lib, dk, tile, parts, C, strength):
    """Each stripe layout's per-channel scan (waves x channel groups x runs),
    with two segments so the state pass and its composition run too; "strong"
    puts chunks beyond the split's range in, so the exact pass runs as well."""
    la = gpu_lib
    B, H, L, dv = 1, 2, 5 * C + 7, 128
    c = W.RandomCase(B, H, L, dk, dv, torch.bfloat16, W.PHI_ELU1 if dk == 64 else 0,
                     W.DECAY_CHANNEL, seed=600 + dk + tile + parts + C, scale=1.0 / np.sqrt(dk),
                     channel_mean=0.3, with_state=True)
    q, k, v, decay, S0 = W.random_inputs(c)
    if strength == "strong":
        decay = _strong_log_decay("mixed", B, H, L, dk, seed=601)
        decay[:, 0, C:2 * C] = -9.0
    print(f"[channel scan layout] dk={dk} tile={tile} parts={parts} C={C} {strength}", flush=True)
    with la.using_plan(la.KERNEL_STRIPE, tile, 2, parts, 0):
        got = la.plan(B, H, L, dk, dv, C, decay_kind=W.DECAY_CHANNEL)
        assert got[:4] == (la.KERNEL_STRIPE, tile, 2, parts), got
        S = S0.to(DEV).contiguous()
        out = la.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=C, phi=c.phi,
                           decay_kind=W.DECAY_CHANNEL, decay=decay.to(DEV).contiguous(), state=S)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(S).all()
    ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), c.phi, W.DECAY_CHANNEL, _np(decay),
                                  _np(S0))
    e = (oracle.rel_err(_np(out), ref), oracle.rel_err(_np(S), ref_s))
    print(f"[channel scan layout] dk={dk} tile={tile} parts={parts} C={C} {strength}: "
          f"out/state rel err {e}", flush=True)
    assert e[0] <= 1e-2 and e[1] <= 1e-2
