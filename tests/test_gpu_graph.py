"""HIP-graph capture of the library's calls.

`la_state_init` clears with a fill kernel (no memset node) and `la_chunk_fwd`
and `la_decode_step` only enqueue kernels on the given stream, so a step made
of them can be captured once and replayed.  Every replay, with eager work and
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
