"""The full-size workloads on the GPU, in the launch configuration the bench times.

Each workload runs whole on the GPU (all heads, full length, default plan);
the fp64 oracle then recomputes a few sampled heads token by token and the
sampled output rows and final states must match within the bar for bf16
inputs (max|err| / max|ref| <= 1e-2).
"""
import numpy as np
import pytest
import torch

import oracle
from chunkwise_recurrence_amd import workloads as W

pytestmark = pytest.mark.gpu

SAMPLED_HEADS = {"elu_bf16": [0, 17, 38, 63], "retnet_bf16": [0, 31, 32, 63],
                 "gated_bf16": [0, 5, 15]}


def _np(t):
    return t.detach().to("cpu", torch.float64).numpy()


@pytest.mark.parametrize("name", ["elu_bf16", "retnet_bf16", "gated_bf16"])
def test_workload_sampled_heads(gpu_lib, name):
    la = gpu_lib
    w = W.WORKLOADS[name]
    print(f"[workload] {name} B={w.B} H={w.H} L={w.L} d={w.dk} C={w.C} plan={la.plan(w.B, w.H, w.L, w.dk, w.dv, w.C)}",
          flush=True)
    q, k, v, decay = W.chunk_inputs(w)
    dev = torch.device("cuda:0")
    S = torch.zeros(w.B, w.H, w.dk, w.dv, device=dev)
    out = la.chunk_fwd(q.to(dev), k.to(dev), v.to(dev), C=w.C, phi=w.phi, decay_kind=w.decay_kind,
                       decay=None if decay is None else decay.to(dev), state=S)
    torch.cuda.synchronize()
    heads = SAMPLED_HEADS[name]
    flat = lambda x: x.reshape(w.B * w.H, *x.shape[2:])  # noqa: E731
    qs, ks, vs = (flat(x)[heads][None] for x in (q, k, v))
    if decay is None:
        ds = None
    elif w.decay_kind == W.DECAY_HEAD:
        ds = decay  # gamma[H]; remapped below per head
    else:
        ds = flat(decay)[heads][None]
    if w.decay_kind == W.DECAY_HEAD:
        # every sampled head keeps its own gamma: run the oracle head by head
        refs, ref_ss = [], []
        for i, bh in enumerate(heads):
            h = bh % w.H
            r, rs = oracle.recurrent(_np(qs[:, i:i + 1]), _np(ks[:, i:i + 1]), _np(vs[:, i:i + 1]),
                                     w.phi, W.DECAY_HEAD, np.array([float(decay[h])]))
            refs.append(r)
            ref_ss.append(rs)
        ref = np.concatenate(refs, axis=1)
        ref_s = np.concatenate(ref_ss, axis=1)
    else:
        ref, ref_s = oracle.recurrent(_np(qs), _np(ks), _np(vs), w.phi, w.decay_kind,
                                      None if ds is None else _np(ds))
    got = _np(flat(out.cpu())[heads][None])
    got_s = _np(flat(S.cpu())[heads][None])
    e_out, e_s = oracle.rel_err(got, ref), oracle.rel_err(got_s, ref_s)
    print(f"{name}: sampled heads {heads}: output rel err {e_out:.3e}, state rel err {e_s:.3e}")
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


def test_decode_workload_sampled_heads(gpu_lib):
    """256 sequences x 32 heads, fp32 state 0.01 N(0,1), 1000 bf16 steps; the oracle follows
    four sampled heads through all 1000 steps."""
    la = gpu_lib
    w = W.DECODE
    stream = W.DecodeStream(w)
    S0 = stream.initial_state()
    dev = torch.device("cuda:0")
    S = S0.to(dev)
    picks = [(0, 0), (17, 5), (128, 31), (255, 16)]
    ref_S = np.stack([_np(S0[n, h]) for n, h in picks])[None]
    worst = 0.0
    for t in range(w.steps):
        q, k, v = stream.step()
        o = la.decode_step(q.to(dev, non_blocking=True), k.to(dev, non_blocking=True),
                           v.to(dev, non_blocking=True), S)
        if t % 100 == 99 or t == w.steps - 1:
            print(f"decode step {t + 1}/{w.steps}", flush=True)
        sel = lambda x: np.stack([_np(x[n, h]) for n, h in picks])[None]  # noqa: E731
        ro, ref_S = oracle.decode_step(sel(q), sel(k), sel(v), state=ref_S)
        if t % 50 == 0 or t == w.steps - 1:
            got = np.stack([_np(o[n, h]) for n, h in picks])[None]
            worst = max(worst, oracle.rel_err(got, ro))
    torch.cuda.synchronize()
    got_S = np.stack([_np(S[n, h]) for n, h in picks])[None]
    e_s = oracle.rel_err(got_S, ref_S)
    print(f"decode: worst sampled output rel err {worst:.3e}, state rel err {e_s:.3e}")
    assert worst <= 1e-2 and e_s <= 1e-4


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
