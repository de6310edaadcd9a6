"""HIP-graph capture of the library's calls.

`la_state_init` clears with a fill kernel (no memset node), and `la_chunk_fwd`,
`la_chunk_fwd_norm`, `la_delta_fwd` and `la_decode_step` only enqueue kernels
on the given stream, so a step made of them can be captured once and replayed.  Every replay, with eager work and
synchronisation between replays, must give the eager result bit for bit (the
same kernels on the same inputs), and the eager result must match the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from chunkwise_recurrence_amd import workloads as W

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().to("cpu", torch.float64).numpy()


@pytest.mark.parametrize("kind", [W.DECAY_HEAD, W.DECAY_GATE])
def test_forward_step_replays_like_eager(gpu_lib, kind):
    la = gpu_lib
    dev = torch.device("cuda:0")
    # 4 heads of 21 chunks (ragged last): the plan splits the sequence, so the
    # step holds the fill, the segment state pass and the output pass
    c = W.RandomCase(1, 4, 64 * 20 + 17, 128, 128, torch.bfloat16, W.PHI_IDENTITY, kind,
                     seed=900 + kind, scale=1.0 / np.sqrt(128), gate_shift=-4.0)
    q, k, v, d, _ = W.random_inputs(c)
    assert la.plan(c.B, c.H, c.L, c.dk, c.dv, 64)[2] > 1
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    d = d.to(dev, torch.float32).contiguous()
    S = torch.empty(c.B, c.H, c.dk, c.dv, device=dev)
    out = torch.empty_like(v)
    need = la.chunk_fwd_workspace_bytes(c.B, c.H, c.L, c.dk, c.dv, 64, la.LA_BF16, kind)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def step(stream):
        la.state_init(S, stream=stream)
        la.chunk_fwd(q, k, v, C=64, phi=W.PHI_IDENTITY, decay_kind=kind, decay=d, state=S,
                     out=out, workspace=ws, stream=stream)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref_o, ref_s = out.clone(), S.clone()
    o64, s64 = oracle.recurrent(_np(q), _np(k), _np(v), W.PHI_IDENTITY, kind, _np(d),
                                np.zeros((c.B, c.H, c.dk, c.dv)))
    assert oracle.rel_err(_np(ref_o), o64) <= 1e-2
    assert oracle.rel_err(_np(ref_s), s64) <= 1e-2

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            step(side)
    torch.cuda.synchronize()
    for i in range(4):
        # eager work between replays: scribble over everything the step writes
        out.fill_(float(i + 1))
        S.fill_(-1.0)
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"replay {i}: output differs from the eager call"
        assert torch.equal(S, ref_s), f"replay {i}: final state differs from the eager call"


def test_decode_steps_replay_like_eager(gpu_lib):
    la = gpu_lib
    dev = torch.device("cuda:0")
    N, H, d, n = 8, 4, 128, 5
    g0 = torch.Generator().manual_seed(950)
    S0 = (torch.randn(N, H, d, d, generator=g0) * 0.01).to(dev)
    qs = [(torch.randn(N, H, d, generator=g0) / np.sqrt(d)).to(torch.bfloat16).to(dev)
          for _ in range(3 * n)]
    S = S0.clone()
    out = torch.empty(N, H, d, dtype=torch.bfloat16, device=dev)
    outs = torch.empty(n, N, H, d, dtype=torch.bfloat16, device=dev)

    def steps(stream):
        for t in range(n):
            la.decode_step(qs[3 * t], qs[3 * t + 1], qs[3 * t + 2], state=S, out=out,
                           stream=stream)
            outs[t].copy_(out)

    steps(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref_outs, ref_s = outs.clone(), S.clone()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        S.copy_(S0)
        steps(side)
        torch.cuda.synchronize()
        S.copy_(S0)
        with torch.cuda.graph(g, stream=side):
            steps(side)
    torch.cuda.synchronize()
    for i in range(3):
        S.copy_(S0)
        outs.fill_(float(i))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, ref_outs), f"replay {i}: outputs differ from the eager steps"
        assert torch.equal(S, ref_s), f"replay {i}: state differs from the eager steps"


def _capture_and_replay(step, results, scribble, replays=4):
    """Run `step` eagerly, capture it on a side stream and replay it `replays`
    times with `scribble(i)` (eager overwrites of what the step writes) before
    each replay; every replay must reproduce the eager `results` bit for bit."""
    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    refs = [t.clone() for t in results]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            step(side)
    torch.cuda.synchronize()
    for i in range(replays):
        scribble(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (t, r) in enumerate(zip(results, refs)):
            assert torch.equal(t, r), f"replay {i}: result {j} differs from the eager call"
    return refs


def test_normalised_step_replays_like_eager(gpu_lib):
    """The normalised form with z_0 given: the step also holds the z_0 copy
    kernel, since the plan splits the sequence into segments."""
    la = gpu_lib
    dev = torch.device("cuda:0")
    c = W.RandomCase(1, 4, 64 * 20 + 17, 128, 128, torch.bfloat16, W.PHI_ELU1, W.DECAY_HEAD,
                     seed=960, scale=1.0 / np.sqrt(128))
    q, k, v, d, _ = W.random_inputs(c)
    assert la.plan(c.B, c.H, c.L, c.dk, c.dv, 64)[2] > 1
    z0 = torch.rand(c.B, c.H, c.dk, generator=torch.Generator().manual_seed(961)) * 4.0 + 0.5
    S0 = torch.randn(c.B, c.H, c.dk, c.dv, generator=torch.Generator().manual_seed(962)) * 0.1
    q, k, v, d = q.to(dev), k.to(dev), v.to(dev), d.to(dev).contiguous()
    S, z = torch.empty(c.B, c.H, c.dk, c.dv, device=dev), torch.empty(c.B, c.H, c.dk, device=dev)
    out = torch.empty_like(v)
    need = la.chunk_fwd_workspace_bytes(c.B, c.H, c.L, c.dk, c.dv, 64, la.LA_BF16, c.decay_kind)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    S0d, z0d = S0.to(dev), z0.to(dev)

    def step(stream):
        S.copy_(S0d)
        z.copy_(z0d)
        la.chunk_fwd(q, k, v, C=64, phi=c.phi, decay_kind=c.decay_kind, decay=d, state=S,
                     out=out, workspace=ws, stream=stream, normalize=True, norm_state=z)

    def scribble(i):
        out.fill_(float(i + 1))
        S.fill_(-1.0)
        z.fill_(-2.0)
        ws.fill_(0x5A)

    ro, rs, rz = _capture_and_replay(step, [out, S, z], scribble)
    o64, s64, z64 = oracle.recurrent(_np(q), _np(k), _np(v), c.phi, c.decay_kind, _np(d),
                                     S0.double().numpy(), normalize=True,
                                     norm_state=z0.double().numpy())
    for x, r in ((ro, o64), (rs, s64), (rz, z64)):
        assert oracle.rel_err(_np(x), r) <= 1e-2


def test_channel_gate_step_replays_like_eager(gpu_lib):
    la = gpu_lib
    dev = torch.device("cuda:0")
    c = W.RandomCase(1, 4, 64 * 20 + 17, 128, 128, torch.bfloat16, W.PHI_IDENTITY,
                     W.DECAY_CHANNEL, seed=970, scale=1.0 / np.sqrt(128), channel_mean=0.8)
    q, k, v, d, _ = W.random_inputs(c)
    q, k, v, d = q.to(dev), k.to(dev), v.to(dev), d.to(dev).contiguous()
    S = torch.empty(c.B, c.H, c.dk, c.dv, device=dev)
    out = torch.empty_like(v)
    need = la.chunk_fwd_workspace_bytes(c.B, c.H, c.L, c.dk, c.dv, 64, la.LA_BF16, c.decay_kind)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def step(stream):
        la.state_init(S, stream=stream)
        la.chunk_fwd(q, k, v, C=64, phi=c.phi, decay_kind=c.decay_kind, decay=d, state=S,
                     out=out, workspace=ws, stream=stream)

    def scribble(i):
        out.fill_(float(i + 1))
        S.fill_(-1.0)
        ws.fill_(0xA5)

    ro, rs = _capture_and_replay(step, [out, S], scribble)
    o64, s64 = oracle.recurrent(_np(q), _np(k), _np(v), c.phi, c.decay_kind, _np(d),
                                np.zeros((c.B, c.H, c.dk, c.dv)))
    assert oracle.rel_err(_np(ro), o64) <= 1e-2
    assert oracle.rel_err(_np(rs), s64) <= 1e-2


def test_delta_step_replays_like_eager(gpu_lib):
    """Gated DeltaNet: the step holds the preparation kernel, the chunk
    recurrence and the output pass, all on the capture stream."""
    la = gpu_lib
    dev = torch.device("cuda:0")
    c = W.RandomCase(1, 4, 64 * 20 + 17, 128, 128, torch.bfloat16, W.PHI_IDENTITY,
                     W.DECAY_GATE, seed=980, scale=1.0 / np.sqrt(128), gate_shift=-4.0)
    q, k, v, beta, d, _ = W.random_delta_inputs(c)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    beta, d = beta.to(dev).contiguous(), d.to(dev).contiguous()
    S = torch.empty(c.B, c.H, c.dk, c.dv, device=dev)
    out = torch.empty_like(v)
    need = la.delta_fwd_workspace_bytes(c.B, c.H, c.L, c.dk, c.dv, 64, la.LA_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def step(stream):
        la.state_init(S, stream=stream)
        la.delta_fwd(q, k, v, beta, C=64, decay_kind=c.decay_kind, decay=d, state=S, out=out,
                     workspace=ws, stream=stream)

    def scribble(i):
        out.fill_(float(i + 1))
        S.fill_(-1.0)
        ws.fill_(0xA5)

    ro, rs = _capture_and_replay(step, [out, S], scribble)
    o64, s64 = oracle.delta_recurrent(_np(q), _np(k), _np(v), _np(beta), c.decay_kind, _np(d),
                                      np.zeros((c.B, c.H, c.dk, c.dv)))
    assert oracle.rel_err(_np(ro), o64) <= 1e-2
    assert oracle.rel_err(_np(rs), s64) <= 1e-2
