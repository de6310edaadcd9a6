"""Benchmark: chunked-forward tokens/s at L = 16K, d = 128, bf16 (per-head RetNet
decay), plus decode steps/s, each against the MI355X HBM roofline, and the
fp64 CPU oracle timed on a bounded sample as a reported baseline.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps N] [--no-cpu]

Prints ONE JSON line.  A step is one la_chunk_fwd over the whole workload
(B=2, H=32, L=16384, d_k=d_v=128, C=64, bf16, gamma_h = linspace(0.9, 0.999)),
inputs resident in HBM.  The dominant kernel's duration is measured with HIP
events on the stream the library launches on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
BF16_PEAK_TFLOPS = 2500.0      # MI355X published dense bf16 MFMA
# Counter results for the timed forward, from rocprofv3 --pmc passes over
# `python bench.py --profile`: HBM traffic (FETCH_SIZE / WRITE_SIZE scaled by a
# copy kernel of known size) and MFMA busy time.  Each file records the sha256
# of the library sources it was measured on and is used only while they match.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "bench_legs_hbm_traffic.md")
MFMA_PROFILE = os.path.join(ROOT, "profiles", "bench_legs_mfma.md")
COPY_BYTES = 1 << 29           # the calibration copy: 512 MiB read, 512 MiB written


def kernel_source_digest() -> str:
    """sha256 over the library's sources (kernels, C ABI, header)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "chunkwise_recurrence_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "la.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profile_value(path: str, key: str):
    """A `- key: value` field of a committed profile summary, or None when the
    file is missing or was measured on other library sources."""
    try:
        text = open(path).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != kernel_source_digest():
        return None
    try:
        return float(fields[key])
    except (KeyError, ValueError):
        return None


def chunk_algorithmic(w, with_state: bool):
    """Minimal bytes and the method's flops of one forward over workload w."""
    ht = w.B * w.H * w.L
    esz = 2 if str(w.dtype).endswith("bfloat16") else 4
    by = ht * (2 * w.dk + 2 * w.dv) * esz          # read q, k, v; write o
    if w.decay_kind in (2, 3):
        by += ht * 4                               # per-token decay data
    elif w.decay_kind == 4:
        by += ht * w.dk * 4                        # per-channel log decay
    elif w.decay_kind == 1:
        by += w.H * 4
    if with_state:
        by += 2 * w.B * w.H * w.dk * w.dv * 4      # read S_0, write S_L
    # QK^T (2 C d_k) + P.V (2 C d_v) + Q S (2 d_k d_v) + K^T V (2 d_k d_v) per head-token
    flops = ht * (2 * w.C * w.dk + 2 * w.C * w.dv + 4 * w.dk * w.dv)
    return by, flops


SETTLE_S = 0.1  # seconds of untimed steps before each forward leg's warm-up


def settle(torch, fn):
    """Run fn untimed for SETTLE_S seconds of wall time.  The inputs of each leg
    are drawn on the CPU, during which the GPU idles and lowers its clocks; it
    takes some milliseconds of work to bring them back, longer than a few
    warm-up steps last, so without this the first timed steps run slow."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def fresh_memory(torch):
    """Return the blocks earlier legs freed to the device before a leg draws its
    inputs, so that every leg's buffers come from fresh allocations as in a
    process of its own: the delta leg ran 5 % slower (0.80 against 0.76 ms) in
    some runs whose inputs and workspace reused the caching allocator's blocks
    from the legs before it; the other legs time the same either way."""
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def bench_chunk(la, torch, W, steps, warmup):
    fresh_memory(torch)
    w = W.WORKLOADS["retnet_bf16"]
    dev = torch.device("cuda:0")
    q, k, v, gamma = W.chunk_inputs(w)
    q, k, v, gamma = q.to(dev), k.to(dev), v.to(dev), gamma.to(dev)
    S = torch.zeros(w.B, w.H, w.dk, w.dv, device=dev)
    out = torch.empty_like(v)
    need = la.chunk_fwd_workspace_bytes(w.B, w.H, w.L, w.dk, w.dv, w.C, la.LA_BF16, w.decay_kind)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        la.state_init(S, stream=stream)
        la.chunk_fwd(q, k, v, C=w.C, phi=w.phi, decay_kind=w.decay_kind, decay=gamma, state=S,
                     out=out, workspace=ws if need else None, stream=stream)

    settle(torch, step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # whole-step timing
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / steps
    # the forward kernel(s) alone, bracketed by events on the launch stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        la.state_init(S, stream=stream)
        a.record(stream)
        la.chunk_fwd(q, k, v, C=w.C, phi=w.phi, decay_kind=w.decay_kind, decay=gamma, state=S,
                     out=out, workspace=ws if need else None, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    kern_ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    by, flops = chunk_algorithmic(w, with_state=True)
    kernel, tile, P, groups, split = la.plan(w.B, w.H, w.L, w.dk, w.dv, w.C)
    return dict(w=w, ms_step=ms_step, wall=wall, kern_ms=kern_ms, bytes=by, flops=flops,
                kernel=kernel, tile=tile, P=P, groups=groups, split=split, need=need)


SCRUB_BYTES = 1 << 29  # a cold call is preceded by a 512 MiB write (the MALL holds 256 MB)


def bench_forward_leg(la, torch, W, name, steps, warmup, cold=False):
    """la_chunk_fwd on workload `name` (state init outside the timing), each call
    bracketed by HIP events on the launch stream.  cold: before every call a
    512 MiB buffer is written, so the inputs are not served from the memory-side
    cache (elu_bf16's 100 MB of inputs fit in it)."""
    fresh_memory(torch)
    w = W.WORKLOADS[name]
    dev = torch.device("cuda:0")
    q, k, v, decay = W.chunk_inputs(w)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    decay = None if decay is None else decay.to(dev)
    S = torch.zeros(w.B, w.H, w.dk, w.dv, device=dev)
    out = torch.empty_like(v)
    need = la.chunk_fwd_workspace_bytes(w.B, w.H, w.L, w.dk, w.dv, w.C, la.LA_BF16, w.decay_kind)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    scrub = torch.empty(SCRUB_BYTES, dtype=torch.uint8, device=dev) if cold else None

    def call():
        la.chunk_fwd(q, k, v, C=w.C, phi=w.phi, decay_kind=w.decay_kind, decay=decay, state=S,
                     out=out, workspace=ws if need else None, stream=stream)

    settle(torch, call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i, (a, b) in enumerate(ev):
        la.state_init(S, stream=stream)
        if cold:
            scrub.fill_(i & 0xFF)
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    by, flops = chunk_algorithmic(w, with_state=True)
    return dict(w=w, ms=ms, bytes=by, flops=flops, plan=la.plan(w.B, w.H, w.L, w.dk, w.dv, w.C))


def leg_report(r, tokens, profile_key=None, plan=None):
    """The per-leg JSON object: time, tokens/s and the roofline block (algorithmic
    bytes / HIP-event time against 8 TB/s; counter traffic and MFMA busy from
    profiles/ while their sources match)."""
    ach = r["bytes"] / (r["ms"] / 1000.0) / 1e9
    rep = {"ms_per_call": r["ms"], "tokens_per_s": tokens / (r["ms"] / 1000.0),
           "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": ach / HBM_PEAK_GBS, "algorithmic_bytes": r["bytes"],
                        "traffic": None if profile_key is None else
                        profile_value(TRAFFIC_PROFILE, f"hbm_bytes_{profile_key}"),
                        "rocprof_mfma_busy_pct": None if profile_key is None else
                        profile_value(MFMA_PROFILE, f"mfma_busy_pct_{profile_key}")}}
    if "flops" in r:
        tf = r["flops"] / (r["ms"] / 1000.0) / 1e12
        rep["roofline"]["mfma_tflops"] = tf
        rep["roofline"]["mfma_frac"] = tf / BF16_PEAK_TFLOPS
    if plan is not None:
        rep["plan"] = plan
    return rep


def bench_chunk_norm(la, torch, W, steps, warmup):
    """The normalised form (la_chunk_fwd_norm) on the timed workload's shapes,
    with phi = elu + 1 so that every denominator is positive."""
    fresh_memory(torch)
    w = W.WORKLOADS["retnet_bf16"]
    dev = torch.device("cuda:0")
    q, k, v, gamma = W.chunk_inputs(w)
    q, k, v, gamma = q.to(dev), k.to(dev), v.to(dev), gamma.to(dev)
    S = torch.zeros(w.B, w.H, w.dk, w.dv, device=dev)
    z = torch.zeros(w.B, w.H, w.dk, device=dev)
    out = torch.empty_like(v)
    need = la.chunk_fwd_workspace_bytes(w.B, w.H, w.L, w.dk, w.dv, w.C, la.LA_BF16, w.decay_kind)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        la.chunk_fwd(q, k, v, C=w.C, phi=la.PHI_ELU1, decay_kind=w.decay_kind, decay=gamma,
                     state=S, out=out, workspace=ws if need else None, stream=stream,
                     normalize=True, norm_state=z)

    settle(torch, call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    by, _ = chunk_algorithmic(w, with_state=True)
    by += 2 * w.B * w.H * w.dk * 4                 # read z_0, write z_L
    return dict(w=w, ms=ms, bytes=by)


def bench_chunk_gla(la, torch, W, steps, warmup):
    """The per-channel (GLA) gate on its workload: la_chunk_fwd with log a
    given per token, head and key channel."""
    fresh_memory(torch)
    w = W.WORKLOADS["gla_bf16"]
    dev = torch.device("cuda:0")
    q, k, v, log_a = W.chunk_inputs(w)
    q, k, v, log_a = q.to(dev), k.to(dev), v.to(dev), log_a.to(dev)
    S = torch.zeros(w.B, w.H, w.dk, w.dv, device=dev)
    out = torch.empty_like(v)
    need = la.chunk_fwd_workspace_bytes(w.B, w.H, w.L, w.dk, w.dv, w.C, la.LA_BF16, w.decay_kind)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        la.chunk_fwd(q, k, v, C=w.C, phi=w.phi, decay_kind=w.decay_kind, decay=log_a, state=S,
                     out=out, workspace=ws if need else None, stream=stream)

    settle(torch, call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    by, flops = chunk_algorithmic(w, with_state=True)
    return dict(w=w, ms=ms, bytes=by, flops=flops)


def bench_delta(la, torch, W, steps, warmup):
    """The delta rule (Gated DeltaNet) on delta_bf16: la_delta_fwd, both passes."""
    fresh_memory(torch)
    w = W.DELTA
    dev = torch.device("cuda:0")
    q, k, v, beta, g = W.delta_inputs(w)
    q, k, v, beta, g = q.to(dev), k.to(dev), v.to(dev), beta.to(dev), g.to(dev)
    S = torch.zeros(w.B, w.H, w.dk, w.dv, device=dev)
    out = torch.empty_like(v)
    ws = torch.empty(la.delta_fwd_workspace_bytes(w.B, w.H, w.L, w.dk, w.dv, w.C, la.LA_BF16),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        la.delta_fwd(q, k, v, beta, C=w.C, decay_kind=w.decay_kind, decay=g, state=S, out=out,
                     workspace=ws, stream=stream)

    settle(torch, call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    by, _ = chunk_algorithmic(w, with_state=True)
    by += w.B * w.H * w.L * 4                      # beta
    return dict(w=w, ms=ms, bytes=by)


def bench_decode(la, torch, W, steps, reps=3):
    fresh_memory(torch)
    w = W.DECODE
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(w.seed)
    S0 = torch.randn((w.N, w.H, w.dk, w.dv), generator=g, device=dev) * w.state_std
    S = S0.clone()
    qkv = torch.randn((steps, 3, w.N, w.H, w.dk), generator=g, device=dev) * w.scale
    qkv = qkv.to(torch.bfloat16)
    out = torch.empty((w.N, w.H, w.dv), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def run():
        for t in range(steps):
            la.decode_step(qkv[t, 0], qkv[t, 1], qkv[t, 2], S, out=out, stream=stream)

    run()  # warm-up pass (also compiles nothing: the library is precompiled)
    S.copy_(S0)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        S.copy_(S0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = sorted(times)[len(times) // 2]
    per_step_bytes = w.N * w.H * (2 * w.dk * w.dv * 4 + (2 * w.dk + 2 * w.dv) * 2)
    return dict(w=w, steps=steps, ms=ms, step_us=1000.0 * ms / steps, bytes=per_step_bytes)


CPU_BUDGET_S = 6.0  # seconds of oracle work per config in the CPU baseline


def _oracle_chunk_rate(W, name, cores):
    """Oracle tokens/s on workload `name`: the whole batch when it fits the budget
    (calibrated on one head), else the first heads that do, scaled to the batch."""
    import oracle
    w = W.WORKLOADS[name]
    heads_all = w.B * w.H
    f64 = lambda t: None if t is None else t.double().numpy()  # noqa: E731

    def args_for(n):
        q, k, v, d = W.chunk_inputs(w, heads=slice(0, n))
        if w.decay_kind == 1:
            # gamma[h] of the first n flattened heads, one per head of a [1, n] batch
            dec = f64(d)[[bh % w.H for bh in range(n)]]
        else:
            dec = f64(d)
            if dec is not None:
                dec = dec[None]
        return (f64(q)[None], f64(k)[None], f64(v)[None], w.phi, w.decay_kind, dec)

    a1 = args_for(1)
    t0 = time.perf_counter()
    oracle.recurrent(*a1, nthreads=1)
    one = time.perf_counter() - t0
    n = max(1, min(heads_all, int(CPU_BUDGET_S / max(one, 1e-4)) * cores))
    a = args_for(n)
    t0 = time.perf_counter()
    oracle.recurrent(*a, nthreads=cores)
    el = time.perf_counter() - t0
    used = min(cores, n)
    # a token (b, t) carries H head-tokens; the sample held n * L head-tokens
    rate = n * w.L / el / w.H
    return rate, used, (f"{n} of {heads_all} heads x L={w.L} of the {name} workload, fp64 token "
                        f"by token in {el:.2f} s on {used} threads; scaled to tokens/s of the "
                        f"whole batch")


def _oracle_decode_rate(W, cores, sequences=32):
    """Oracle decode steps/s: `sequences` of the 256 sequences (x 32 heads), drawn
    with the decode workload's recipe, through all its steps -- the oracle's
    decode step is one token of the recurrence, so the steps of a head run as
    one recurrence -- scaled to steps/s of all 256 x 32 heads."""
    import oracle
    w = W.DECODE
    st = W.DecodeStream(w, N=sequences)
    S0 = st.initial_state().double().numpy()
    qkv = [st.step() for _ in range(w.steps)]
    q, k, v = (torch_stack_steps([x[i] for x in qkv]) for i in range(3))
    t0 = time.perf_counter()
    oracle.recurrent(q, k, v, state=S0, nthreads=cores)
    el = time.perf_counter() - t0
    frac = sequences / w.N
    return w.steps * frac / el, min(cores, sequences * w.H), (
        f"{sequences} of {w.N} sequences x {w.H} heads x {w.steps} steps of decode_bf16, fp64 in "
        f"{el:.2f} s; scaled to steps/s of all {w.N * w.H} heads")


def torch_stack_steps(xs):
    """[T] list of [N, H, d] step tensors -> fp64 [N, H, T, d]."""
    import torch
    return torch.stack(xs, dim=2).double().numpy()


def cpu_baseline(W):
    """The fp64 oracle on every timed workload, on all host cores: the headline
    (retnet_bf16) as the baseline proper, the others under `configs`."""
    import oracle
    cores = oracle.host_threads()
    rate, used, sample = _oracle_chunk_rate(W, "retnet_bf16", cores)
    res = {"value": rate, "unit": "tokens/s", "cores": used, "kind": "oracle", "sample": sample,
           "configs": {}}
    for name in ("elu_bf16", "gated_bf16"):
        r, u, smp = _oracle_chunk_rate(W, name, cores)
        res["configs"][name] = {"value": r, "unit": "tokens/s", "cores": u, "sample": smp}
    r, u, smp = _oracle_decode_rate(W, cores)
    res["configs"]["decode_bf16"] = {"value": r, "unit": "steps/s", "cores": u, "sample": smp}
    return res


def profile_pass(la, torch, W):
    """A short fixed sequence of launches for counter passes: one plain copy of
    COPY_BYTES (the calibration), then the forward of the timed workload
    (state init + la_chunk_fwd) three times, 20 decode steps, three forwards
    each of elu_bf16 and gated_bf16, two of the normalised form, two of the
    per-channel gate workload, then two delta-rule forwards."""
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    bench_chunk(la, torch, W, steps=1, warmup=1)
    bench_decode(la, torch, W, steps=20, reps=1)
    bench_forward_leg(la, torch, W, "elu_bf16", steps=2, warmup=1)
    bench_forward_leg(la, torch, W, "gated_bf16", steps=2, warmup=1)
    bench_chunk_norm(la, torch, W, steps=1, warmup=1)
    bench_chunk_gla(la, torch, W, steps=1, warmup=1)
    bench_delta(la, torch, W, steps=1, warmup=1)
    torch.cuda.synchronize()
    print(json.dumps({"profile_pass": True, "copy_bytes": COPY_BYTES,
                      "source_sha256": kernel_source_digest()}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="run the fixed launch sequence for rocprofv3 counter passes instead")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: every head and every decode sequence is "
              "independent, so N GPUs would each run this same kernel on 1/N of the heads "
              "and only the one-GPU run is measured.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import chunkwise_recurrence_amd as la
    from chunkwise_recurrence_amd import workloads as W
    la.load()
    if args.profile:
        # counter passes want a short, fixed launch sequence: no settle phase
        global SETTLE_S
        SETTLE_S = 0.0
        profile_pass(la, torch, W)
        return
    c = bench_chunk(la, torch, W, args.steps, args.warmup)
    e_warm = bench_forward_leg(la, torch, W, "elu_bf16", args.steps, args.warmup)
    e_cold = bench_forward_leg(la, torch, W, "elu_bf16", max(args.steps // 2, 1),
                               max(args.warmup // 2, 1), cold=True)
    gt = bench_forward_leg(la, torch, W, "gated_bf16", args.steps, args.warmup)
    n = bench_chunk_norm(la, torch, W, max(args.steps // 2, 1), max(args.warmup // 2, 1))
    g = bench_chunk_gla(la, torch, W, max(args.steps // 2, 1), max(args.warmup // 2, 1))
    dl = bench_delta(la, torch, W, max(args.steps // 2, 1), max(args.warmup // 2, 1))
    d = bench_decode(la, torch, W, args.decode_steps)
    w = c["w"]
    tokens = w.B * w.L
    value = tokens / (c["ms_step"] / 1000.0)
    achieved = c["bytes"] / (c["kern_ms"] / 1000.0) / 1e9
    dec_gbs = d["bytes"] / (d["step_us"] / 1e6) / 1e9
    res = {
        "metric": "chunked-fwd tokens/sec at L=16K,d=128 bf16; decode steps/s; % MFMA/HBM peak",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": c["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "retnet_bf16", "B": w.B, "H": w.H, "L": w.L, "d_k": w.dk,
                   "d_v": w.dv, "C": w.C, "decay": "per-head gamma = linspace(0.9, 0.999, 32)",
                   "inputs": "q,k,v ~ N(0,1)/sqrt(128) in bf16",
                   "plan": {"kernel": {1: "strip", 2: "stripe"}.get(c["kernel"], c["kernel"]),
                            "dv_tile": c["tile"], "segments": c["P"]}},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": profile_value(TRAFFIC_PROFILE, "hbm_bytes_retnet_bf16"),
                     "kernel": "the chunked forward of one la_chunk_fwd: its segment state pass "
                               "and output pass (HIP events around the call)",
                     "kernel_ms": c["kern_ms"], "algorithmic_bytes": c["bytes"],
                     "mfma_tflops": c["flops"] / (c["kern_ms"] / 1000.0) / 1e12,
                     "mfma_frac": c["flops"] / (c["kern_ms"] / 1000.0) / 1e12 / BF16_PEAK_TFLOPS,
                     "rocprof_mfma_busy_pct": profile_value(MFMA_PROFILE,
                                                            "mfma_busy_pct_retnet_bf16")},
        "elu": dict(workload="elu_bf16: B=4, H=16, L=4096, d=64, phi = elu+1, no decay, C=64",
                    warm=leg_report(e_warm, e_warm["w"].B * e_warm["w"].L, "elu_bf16",
                                    e_warm["plan"]),
                    cold=leg_report(e_cold, e_cold["w"].B * e_cold["w"].L)),
        "gated": dict(workload="gated_bf16: B=1, H=16, L=65536, d=128, a_t = exp(-softplus(g_t)), "
                               "C=64",
                      **leg_report(gt, gt["w"].B * gt["w"].L, "gated_bf16", gt["plan"])),
        "normalized": dict(workload="retnet_bf16 shapes, normalised form, phi = elu+1",
                           **leg_report(n, tokens, "norm_retnet_bf16")),
        "gla": dict(workload="gla_bf16: retnet_bf16 shapes, per-channel gate, "
                             "log a ~ -Exp(mean 0.8) per token, head and key channel",
                    **leg_report(g, tokens, "gla_bf16")),
        "delta": dict(workload="delta_bf16: Gated DeltaNet on the retnet_bf16 shapes, unit keys, "
                               "beta ~ U(0,1), gate g ~ N(0,1), C = 64",
                      **leg_report(dl, tokens, "delta_bf16")),
        "decode": {"workload": "decode_bf16", "N": d["w"].N, "H": d["w"].H, "d": d["w"].dk,
                   "steps": d["steps"], "steps_per_s": 1e6 / d["step_us"],
                   "us_per_step": d["step_us"], "bytes_per_step": d["bytes"],
                   "roofline": {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": dec_gbs / HBM_PEAK_GBS,
                                "algorithmic_bytes": d["bytes"],
                                "traffic": profile_value(TRAFFIC_PROFILE, "hbm_bytes_decode_step")}},
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(W)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
