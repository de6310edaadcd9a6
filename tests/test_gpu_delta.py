"""GPU parity of the delta rule (la_delta_fwd, la_delta_decode_step) against
the fp64 oracle (`oracle.delta_recurrent`): DeltaNet and Gated DeltaNet,
S_t = a_t (S_{t-1} - beta_t k_t (k_t^T S_{t-1})) + beta_t k_t v_t^T, o_t = q_t^T S_t
("Linear / Sparse Attention", delta_rule_recurrent; the tutorial's sections
5.1-5.3).  Keys have unit length, as the pages normalise them.  Bars as for
the other paths: 1e-4 (fp32), 1e-2 (bf16 inputs), max|err| / max|ref|."""
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
    q, k, v, beta, decay, S0 = W.random_delta_inputs(c)
    S0 = S0 if S0 is not None else torch.zeros(c.B, c.H, c.dk, c.dv)
    print(f"[delta case] {label} B={c.B} H={c.H} L={c.L} dk={c.dk} dv={c.dv} C={C} "
          f"dtype={c.dtype} decay={c.decay_kind}", flush=True)
    S = S0.to(DEV).contiguous()
    out = la.delta_fwd(q.to(DEV), k.to(DEV), v.to(DEV), beta.to(DEV), C=C,
                       decay_kind=c.decay_kind,
                       decay=None if decay is None else decay.to(DEV).contiguous(), state=S)
    torch.cuda.synchronize()
    ref, ref_s = oracle.delta_recurrent(_np(q), _np(k), _np(v), _np(beta), c.decay_kind,
                                        _np(decay), _np(S0))
    tol = TOL[c.dtype]
    e = (oracle.rel_err(_np(out), ref), oracle.rel_err(_np(S), ref_s))
    assert e[0] <= tol and e[1] <= tol, f"{label}: out/state rel err {e}"
    return e


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_delta_variants(gpu_lib, dtype, kind):
    """Ragged length (3 chunks of 64 and 23 tokens), an initial state, every decay."""
    c = W.RandomCase(2, 2, 64 * 3 + 23, 64, 64, dtype, W.PHI_IDENTITY, kind, seed=600 + kind,
                     scale=1.0 / np.sqrt(64), with_state=True)
    _run(gpu_lib, c, 64, "variants")


@pytest.mark.parametrize("dk,dv,C", [(16, 16, 16), (32, 128, 32), (128, 32, 64), (128, 128, 64),
                                     (64, 32, 16)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_delta_head_dims_and_chunks(gpu_lib, dk, dv, C, dtype):
    c = W.RandomCase(1, 3, 150, dk, dv, dtype, W.PHI_IDENTITY, W.DECAY_GATE,
                     seed=dk + dv + C + 61, scale=1.0 / np.sqrt(dk), with_state=True)
    _run(gpu_lib, c, C, "head dims")


def test_delta_chunk_size_invariance(gpu_lib):
    la = gpu_lib
    c = W.RandomCase(1, 2, 200, 64, 64, torch.float32, W.PHI_IDENTITY, W.DECAY_LOG, seed=640,
                     scale=1.0 / np.sqrt(64), with_state=True)
    q, k, v, beta, decay, S0 = W.random_delta_inputs(c)
    outs = []
    for C in (16, 32, 64):
        S = S0.to(DEV).contiguous()
        outs.append(_np(la.delta_fwd(q.to(DEV), k.to(DEV), v.to(DEV), beta.to(DEV), C=C,
                                     decay_kind=W.DECAY_LOG, decay=decay.to(DEV), state=S)))
    for o in outs[1:]:
        assert oracle.rel_err(o, outs[0]) <= 1e-5


def test_delta_unit_beta_orthonormal_keys_is_additive(gpu_lib):
    """Check [e] of the pages on the GPU: orthonormal keys and beta = 1 make the
    delta rule the additive one (la_chunk_fwd on the same inputs)."""
    la = gpu_lib
    d = 64
    g = torch.Generator().manual_seed(650)
    Qm, _ = torch.linalg.qr(torch.randn(d, d, generator=g, dtype=torch.float64))
    k = Qm.T.to(torch.float32).reshape(1, 1, d, d).contiguous()
    q = torch.randn(1, 1, d, d, generator=g)
    v = torch.randn(1, 1, d, d, generator=g)
    od = la.delta_fwd(q.to(DEV), k.to(DEV), v.to(DEV), torch.ones(1, 1, d, device=DEV), C=32)
    oa = la.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=32)
    torch.cuda.synchronize()
    assert oracle.rel_err(_np(od), _np(oa)) <= 1e-5


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("kind", [0, 3])
def test_delta_prefill_then_decode(gpu_lib, dtype, kind):
    """la_delta_fwd over L tokens, then n decode steps from its state == the recurrence over L + n."""
    la = gpu_lib
    L, n = 100, 5
    c = W.RandomCase(2, 3, L + n, 32, 64, dtype, W.PHI_IDENTITY, kind, seed=660 + kind,
                     scale=1.0 / np.sqrt(32), with_state=True)
    q, k, v, beta, d, S0 = W.random_delta_inputs(c)
    S = S0.to(DEV).contiguous()
    dd = None if d is None else d.to(DEV)
    pre = la.delta_fwd(q[:, :, :L].contiguous().to(DEV), k[:, :, :L].contiguous().to(DEV),
                       v[:, :, :L].contiguous().to(DEV), beta[:, :, :L].contiguous().to(DEV),
                       C=32, decay_kind=kind,
                       decay=None if dd is None else dd[:, :, :L].contiguous(), state=S)
    steps = []
    for t in range(L, L + n):
        steps.append(la.delta_decode_step(
            q[:, :, t].contiguous().to(DEV), k[:, :, t].contiguous().to(DEV),
            v[:, :, t].contiguous().to(DEV), beta[:, :, t].contiguous().to(DEV), S,
            decay_kind=kind, decay=None if dd is None else dd[:, :, t].contiguous()))
    torch.cuda.synchronize()
    ref, ref_s = oracle.delta_recurrent(_np(q), _np(k), _np(v), _np(beta), kind, _np(d), _np(S0))
    tol = TOL[dtype]
    assert oracle.rel_err(_np(pre), ref[:, :, :L]) <= tol
    got = np.stack([_np(o) for o in steps], axis=2)
    assert oracle.rel_err(got, ref[:, :, L:]) <= tol
    assert oracle.rel_err(_np(S), ref_s) <= tol


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (128, 32), (128, 128)])
def test_delta_decode_head_dims(gpu_lib, dk, dv):
    la = gpu_lib
    N, H, T = 5, 3, 4
    g = torch.Generator().manual_seed(dk * 1000 + dv + 2)
    S0 = torch.randn(N, H, dk, dv, generator=g) * 0.1
    S = S0.to(DEV)
    ref_S = _np(S0)
    for _ in range(T):
        q = torch.randn(N, H, dk, generator=g).to(torch.bfloat16)
        k = W.unit_rows(torch.randn(N, H, dk, generator=g)).to(torch.bfloat16)
        v = torch.randn(N, H, dv, generator=g).to(torch.bfloat16)
        beta = torch.rand(N, H, generator=g)
        gate = torch.randn(N, H, generator=g)
        o = la.delta_decode_step(q.to(DEV), k.to(DEV), v.to(DEV), beta.to(DEV), S,
                                 decay_kind=W.DECAY_GATE, decay=gate.to(DEV))
        torch.cuda.synchronize()
        ro, ref_S = oracle.delta_decode_step(_np(q), _np(k), _np(v), _np(beta), W.DECAY_GATE,
                                             _np(gate), ref_S)
        assert oracle.rel_err(_np(o), ro) < 1e-2
    assert oracle.rel_err(_np(S), ref_S) < 1e-5  # the state itself stays fp32


def test_delta_workload_whole_output(gpu_lib):
    """The full delta_bf16 workload (B=2, H=32, L=16384, d=128, C=64, gated) as the
    bench launches it; the oracle recomputes every head, and the whole output
    and final state are compared."""
    la = gpu_lib
    w = W.DELTA
    print(f"[workload] delta_bf16 B={w.B} H={w.H} L={w.L} d={w.dk} C={w.C}", flush=True)
    q, k, v, beta, decay = W.delta_inputs(w)
    S = torch.zeros(w.B, w.H, w.dk, w.dv, device=DEV)
    out = la.delta_fwd(q.to(DEV), k.to(DEV), v.to(DEV), beta.to(DEV), C=w.C,
                       decay_kind=w.decay_kind, decay=decay.to(DEV), state=S)
    torch.cuda.synchronize()
    got, got_s = _np(out), _np(S)
    del out, S
    ref, ref_s = oracle.delta_recurrent(_np(q), _np(k), _np(v), _np(beta), w.decay_kind,
                                        _np(decay))
    e_out, e_s = oracle.rel_err(got, ref), oracle.rel_err(got_s, ref_s)
    print(f"delta_bf16: all heads: output rel err {e_out:.3e}, state rel err {e_s:.3e}",
          flush=True)
    assert e_out <= 1e-2 and e_s <= 1e-2


# Each layout of the matrix-core sequential pass: (B, H, d_k, d_v) and the layout
# the launch picks for it (bf16, 64-token chunks): 32-column tiles in one group
# once B*H*(d_v/32) >= 512, else the column pass (d_k >= 64: 32-column
# workgroups, two waves each carrying 16 columns' whole chain, four moving the
# tiles) or one 16-column group (d_k = 32).
@pytest.mark.parametrize("B,H,dk,dv,layout", [
    (1, 2, 128, 128, "column pass"), (1, 3, 64, 128, "column pass"),
    (8, 32, 64, 64, "one 32-column group"), (8, 32, 32, 64, "one 32-column group"),
    (1, 3, 32, 64, "one 16-column group"), (2, 2, 32, 32, "one 16-column group")])
def test_delta_sequential_pass_layouts(gpu_lib, B, H, dk, dv, layout):
    c = W.RandomCase(B, H, 64 * 2 + 13, dk, dv, torch.bfloat16, W.PHI_IDENTITY, W.DECAY_GATE,
                     seed=680 + B + H + dk + dv, scale=1.0 / np.sqrt(dk), with_state=True)
    _run(gpu_lib, c, 64, f"sequential pass, {layout}")


@pytest.mark.parametrize("dk,dv,L,with_state", [
    (128, 128, 1, True), (128, 64, 37, False), (64, 32, 64, True), (128, 64, 65, False),
    (64, 128, 128, True), (128, 32, 64 * 5 + 63, True)])
def test_delta_column_pass_lengths(gpu_lib, dk, dv, L, with_state):
    """The column pass (bf16, d_k >= 64, few heads) at one token, one partial
    chunk, exactly one and two chunks, one chunk and a token, and a ragged tail;
    with and without an initial state; 32 to 128 value columns."""
    c = W.RandomCase(1, 2, L, dk, dv, torch.bfloat16, W.PHI_IDENTITY, W.DECAY_GATE,
                     seed=900 + dk + dv + L, scale=1.0 / np.sqrt(dk), with_state=with_state)
    _run(gpu_lib, c, 64, f"column pass L={L}")


def test_delta_many_heads_takes_the_32_column_pass(gpu_lib):
    """B*H*(d_v/32) >= 512 keeps 32-column workgroups in the MFMA pass; the
    smaller cases above run the 16-column ones."""
    c = W.RandomCase(4, 32, 64 * 2 + 5, 128, 128, torch.bfloat16, W.PHI_IDENTITY, W.DECAY_GATE,
                     seed=670, scale=1.0 / np.sqrt(128), with_state=True)
    _run(gpu_lib, c, 64, "32-column pass")


@pytest.mark.parametrize("dtype,dk,dv", [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 64),
                                         (torch.float32, 32, 64)])
def test_delta_degenerate_gates_and_strengths(gpu_lib, dtype, dk, dv):
    """Saturated gates (g = +30: a = e^-30, g = -30: a = 1 to fp32 precision)
    mixed with ordinary ones per token, and write strengths at the ends of
    their range (beta = 0: no write; beta = 1 with a unit key: the key's
    direction is replaced), against the oracle."""
    la = gpu_lib
    B, H, L = 1, 3, 64 * 4 + 21
    g = torch.Generator().manual_seed(700 + dk + dv)
    q = (torch.randn(B, H, L, dk, generator=g) / np.sqrt(dk)).to(dtype)
    kr = torch.randn(B, H, L, dk, generator=g)
    k = (kr / kr.norm(dim=-1, keepdim=True)).to(dtype)
    v = torch.randn(B, H, L, dv, generator=g).to(dtype)
    pick = torch.randint(0, 3, (B, H, L), generator=g)
    beta = torch.where(pick == 0, torch.zeros(B, H, L),
                       torch.where(pick == 1, torch.ones(B, H, L), torch.rand(B, H, L, generator=g)))
    pick = torch.randint(0, 3, (B, H, L), generator=g)
    gate = torch.where(pick == 0, torch.full((B, H, L), 30.0),
                       torch.where(pick == 1, torch.full((B, H, L), -30.0),
                                   torch.randn(B, H, L, generator=g)))
    S0 = torch.randn(B, H, dk, dv, generator=g) * 0.1
    S = S0.to(DEV).contiguous()
    out = la.delta_fwd(q.to(DEV), k.to(DEV), v.to(DEV), beta.to(DEV), C=64,
                       decay_kind=W.DECAY_GATE, decay=gate.to(DEV), state=S)
    torch.cuda.synchronize()
    ref, ref_s = oracle.delta_recurrent(_np(q), _np(k), _np(v), _np(beta), W.DECAY_GATE,
                                        _np(gate), _np(S0))
    assert torch.isfinite(out.float()).all() and torch.isfinite(S).all()
    tol = TOL[dtype]
    e = (oracle.rel_err(_np(out), ref), oracle.rel_err(_np(S), ref_s))
    assert e[0] <= tol and e[1] <= tol, f"out/state rel err {e}"
