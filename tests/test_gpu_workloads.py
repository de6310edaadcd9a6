"""The full-size workloads on the GPU, in the launch configuration the bench times.

Each workload runs whole on the GPU (all heads, full length, default plan);
the fp64 oracle then recomputes every head token by token, and the whole
output and the whole final state must match within the bar for bf16 inputs:
max|err| / max|ref| <= 1e-2 over the entire tensor (the pages' "max
relative difference", CS336 lecture 4 code 1 `demo_two_forms`).
"""
import numpy as np
import pytest
import torch

import oracle
from chunkwise_recurrence_amd import workloads as W

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().to("cpu", torch.float64).numpy()


@pytest.mark.parametrize("name", ["elu_bf16", "retnet_bf16", "gated_bf16"])
def test_workload_whole_output(gpu_lib, name):
    la = gpu_lib
    w = W.WORKLOADS[name]
    print(f"[workload] {name} B={w.B} H={w.H} L={w.L} d={w.dk} C={w.C} "
          f"plan={la.plan(w.B, w.H, w.L, w.dk, w.dv, w.C)}", flush=True)
    q, k, v, decay = W.chunk_inputs(w)
    dev = torch.device("cuda:0")
    S = torch.zeros(w.B, w.H, w.dk, w.dv, device=dev)
    out = la.chunk_fwd(q.to(dev), k.to(dev), v.to(dev), C=w.C, phi=w.phi, decay_kind=w.decay_kind,
                       decay=None if decay is None else decay.to(dev), state=S)
    torch.cuda.synchronize()
    got, got_s = _np(out), _np(S)
    del out, S
    ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), w.phi, w.decay_kind,
                                  None if decay is None else _np(decay))
    e_out, e_s = oracle.rel_err(got, ref), oracle.rel_err(got_s, ref_s)
    print(f"{name}: all {w.B * w.H} heads: output rel err {e_out:.3e}, state rel err {e_s:.3e}",
          flush=True)
    assert e_out <= 1e-2 and e_s <= 1e-2


def test_gated_mild_gate(gpu_lib):
    """The gated workload with g - 5 (a ~ 0.993): the carried state matters across chunks
    and segments, so the segment scan is exercised with non-vanishing decay."""
    la = gpu_lib
    w = W.ChunkWorkload("gated_mild", 1, 4, 16384, 128, 128, 64, torch.bfloat16, 0,
                        W.DECAY_GATE, seed=44, scale=1.0 / np.sqrt(128.0), gate_shift=-5.0)
    q, k, v, decay = W.chunk_inputs(w)
    dev = torch.device("cuda:0")
    S = torch.zeros(w.B, w.H, w.dk, w.dv, device=dev)
    out = la.chunk_fwd(q.to(dev), k.to(dev), v.to(dev), C=64, decay_kind=W.DECAY_GATE,
                       decay=decay.to(dev), state=S)
    torch.cuda.synchronize()
    ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), 0, W.DECAY_GATE, _np(decay))
    e_out, e_s = oracle.rel_err(_np(out.cpu()), ref), oracle.rel_err(_np(S.cpu()), ref_s)
    print(f"gated_mild plan={la.plan(1, 4, 16384, 128, 128, 64)}: out {e_out:.3e} state {e_s:.3e}")
    assert e_out <= 1e-2 and e_s <= 1e-2


def test_decode_workload_whole(gpu_lib):
    """256 sequences x 32 heads, fp32 state 0.01 N(0,1), 1000 bf16 steps: every
    head's output on every step and every head's final state against the oracle,
    which runs the 1000 steps of each head as one recurrence (no decay), in
    blocks of 1024 heads."""
    la = gpu_lib
    w = W.DECODE
    stream = W.DecodeStream(w)
    S0 = stream.initial_state()
    steps = [stream.step() for _ in range(w.steps)]
    qs, ks, vs = (torch.stack([st[i] for st in steps]) for i in range(3))  # [T, N, H, d]
    del steps
    dev = torch.device("cuda:0")
    qd, kd, vd = qs.to(dev), ks.to(dev), vs.to(dev)
    S = S0.to(dev)
    outs = torch.empty((w.steps, w.N, w.H, w.dv), dtype=torch.bfloat16, device=dev)
    print(f"[decode] N={w.N} H={w.H} d={w.dk} steps={w.steps}", flush=True)
    for t in range(w.steps):
        la.decode_step(qd[t], kd[t], vd[t], S, out=outs[t])
    torch.cuda.synchronize()
    print("decode: GPU steps done", flush=True)
    NH, T = w.N * w.H, w.steps
    got = outs.cpu().reshape(T, NH, w.dv)
    got_S = S.cpu().reshape(NH, w.dk, w.dv)
    del qd, kd, vd, outs, S
    S0f = S0.reshape(NH, w.dk, w.dv)
    heads_of = lambda x, sl: _np(x.reshape(T, NH, -1)[:, sl].permute(1, 0, 2))[None]  # noqa: E731
    err = ref_max = err_s = ref_s_max = 0.0
    for first in range(0, NH, 1024):
        sl = slice(first, min(first + 1024, NH))
        ref, ref_S = oracle.recurrent(heads_of(qs, sl), heads_of(ks, sl), heads_of(vs, sl),
                                      state=_np(S0f[sl])[None])
        g = _np(got[:, sl].permute(1, 0, 2))[None]
        err = max(err, float(np.abs(g - ref).max()))
        ref_max = max(ref_max, float(np.abs(ref).max()))
        err_s = max(err_s, float(np.abs(_np(got_S[sl])[None] - ref_S).max()))
        ref_s_max = max(ref_s_max, float(np.abs(ref_S).max()))
        print(f"decode: heads {sl.start}..{sl.stop - 1} compared", flush=True)
    e_out, e_s = err / ref_max, err_s / ref_s_max
    print(f"decode: all {NH} heads x {T} steps: output rel err {e_out:.3e}, "
          f"state rel err {e_s:.3e}", flush=True)
    assert e_out <= 1e-2 and e_s <= 1e-4


@pytest.mark.parametrize("d", [128, 64])
def test_single_long_head_many_segments(gpu_lib, d):
    """One head over 65536 tokens: the plan splits it into 256 segments of four
    chunks, so the last segment composes 255 earlier (decay, increment) pairs;
    a mild gate (a ~ 0.993) keeps the state alive across all of them."""
    la = gpu_lib
    L = 65536
    plan = la.plan(1, 1, L, d, d, 64)
    assert plan[2] == 256, plan
    w = W.ChunkWorkload(f"long_head_{d}", 1, 1, L, d, d, 64, torch.bfloat16, 0, W.DECAY_GATE,
                        seed=45 + d, scale=1.0 / np.sqrt(d), gate_shift=-5.0)
    q, k, v, decay = W.chunk_inputs(w)
    g = torch.Generator().manual_seed(46 + d)
    S0 = torch.randn(1, 1, d, d, generator=g) * 0.1
    dev = torch.device("cuda:0")
    S = S0.to(dev).contiguous()
    out = la.chunk_fwd(q.to(dev), k.to(dev), v.to(dev), C=64, decay_kind=W.DECAY_GATE,
                       decay=decay.to(dev), state=S)
    torch.cuda.synchronize()
    ref, ref_s = oracle.recurrent(_np(q), _np(k), _np(v), 0, W.DECAY_GATE, _np(decay), _np(S0))
    e_out, e_s = oracle.rel_err(_np(out.cpu()), ref), oracle.rel_err(_np(S.cpu()), ref_s)
    print(f"long head d={d} plan={plan}: out {e_out:.3e} state {e_s:.3e}")
    assert e_out <= 1e-2 and e_s <= 1e-2
