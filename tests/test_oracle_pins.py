"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

None of these compares the oracle with a copy of itself.  Each check uses a
different route to the same number: exact rational arithmetic, the fully
parallel masked form with explicit products, the chunkwise form, closed
forms of special cases, library routines (torch's elu and sigmoid, BLAS),
and the values the pages print for their own runs.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from chunkwise_recurrence_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
VARIANTS = [(phi, kind) for phi in (oracle.PHI_IDENTITY, oracle.PHI_ELU1)
            for kind in (oracle.DECAY_NONE, oracle.DECAY_HEAD, oracle.DECAY_LOG,
                         oracle.DECAY_GATE)]


def _case(seed, B, H, L, dk, dv, kind, with_state=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    v = rng.standard_normal((B, H, L, dv))
    if kind == oracle.DECAY_HEAD:
        dec = rng.uniform(0.5, 1.0, H)
    elif kind == oracle.DECAY_LOG:
        dec = -np.abs(rng.standard_normal((B, H, L))) * 0.5
    elif kind == oracle.DECAY_GATE:
        dec = rng.standard_normal((B, H, L))
    else:
        dec = None
    S0 = rng.standard_normal((B, H, dk, dv)) if with_state else None
    return q, k, v, dec, S0


# ---------------------------------------------------------------------------
# exact arithmetic: the definition as a double sum, in rationals
# ---------------------------------------------------------------------------
def _exact_outputs(q, k, v, a, S0):
    """o_t = sum_{s<=t} (prod_{r=s+1..t} a_r)(q_t.k_s) v_s + (prod_{r<=t} a_r) q_t^T S_0,
    evaluated in exact rationals (CS336 lecture 4 code 1, the derivation under
    gated_linear_attention_parallel expands the recurrence into this sum)."""
    L, dk = len(q), len(q[0])
    dv = len(v[0])
    out = []
    for t in range(L):
        o = [Fraction(0)] * dv
        for s in range(t + 1):
            w = Fraction(1)
            for r in range(s + 1, t + 1):
                w *= a[r]
            dot = sum(q[t][i] * k[s][i] for i in range(dk))
            for j in range(dv):
                o[j] += w * dot * v[s][j]
        head = Fraction(1)
        for r in range(t + 1):
            head *= a[r]
        for j in range(dv):
            o[j] += head * sum(q[t][i] * S0[i][j] for i in range(dk))
        out.append(o)
    return out


@pytest.mark.parametrize("kind", [oracle.DECAY_NONE, oracle.DECAY_HEAD, oracle.DECAY_LOG])
def test_recurrent_matches_exact_rational_sum(kind):
    """Small integer inputs and dyadic decays, so every fp64 operation of the
    oracle is exact or within a few ulps of the rational answer."""
    rng = np.random.default_rng(11 + kind)
    L, dk, dv = 9, 3, 4  # dk != dv: a transposed state would not even fit
    q = rng.integers(-3, 4, (L, dk)).astype(np.float64)
    k = rng.integers(-3, 4, (L, dk)).astype(np.float64)
    v = rng.integers(-3, 4, (L, dv)).astype(np.float64)
    S0 = rng.integers(-2, 3, (dk, dv)).astype(np.float64)
    if kind == oracle.DECAY_NONE:
        a = [Fraction(1)] * L
        dec = None
    elif kind == oracle.DECAY_HEAD:
        a = [Fraction(3, 4)] * L
        dec = np.array([0.75])
    else:
        halves = rng.integers(0, 3, L)  # a_t in {1, 1/2, 1/4}
        a = [Fraction(1, 2 ** int(h)) for h in halves]
        dec = np.log(np.array([float(x) for x in a]))[None, None]
    out, S = oracle.recurrent(q[None, None], k[None, None], v[None, None],
                              decay_kind=kind, decay=dec, state=S0[None, None])
    to_f = lambda m: [[Fraction(float(x)) for x in row] for row in m]  # noqa: E731
    exact = _exact_outputs(to_f(q), to_f(k), to_f(v), a, to_f(S0))
    ex = np.array([[float(x) for x in row] for row in exact])
    assert np.max(np.abs(out[0, 0] - ex)) <= 1e-12 * max(1.0, np.max(np.abs(ex)))


# ---------------------------------------------------------------------------
# the three forms the pages give agree (recurrent == parallel == chunkwise)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("phi,kind", VARIANTS)
def test_recurrent_equals_parallel_form(phi, kind):
    B, H, L, dk, dv = 2, 3, 13, 5, 3
    q, k, v, dec, S0 = _case(1, B, H, L, dk, dv, kind)
    out, S = oracle.recurrent(q, k, v, phi, kind, dec, S0)
    a = oracle.decay_multipliers(B, H, L, kind, dec)
    op, Sp = oracle.parallel(q, k, v, a, phi, S0)
    assert oracle.rel_err(out, op) < 1e-13
    assert oracle.rel_err(S, Sp) < 1e-13


@pytest.mark.parametrize("phi,kind", VARIANTS)
def test_recurrent_equals_chunkwise_form(phi, kind):
    """Chunk sizes 1, 4, 7 and L on L = 13 (ragged), d = 6, as in check [a]."""
    B, H, L, dk, dv = 1, 2, 13, 6, 6
    q, k, v, dec, S0 = _case(2, B, H, L, dk, dv, kind)
    out, S = oracle.recurrent(q, k, v, phi, kind, dec, S0)
    a = oracle.decay_multipliers(B, H, L, kind, dec)
    for C in (1, 4, 7, L):
        oc, Sc = oracle.chunkwise(q, k, v, a, C, phi, S0)
        assert oracle.rel_err(out, oc) < 1e-13, C
        assert oracle.rel_err(S, Sc) < 1e-13, C


def test_chunk_size_invariance_of_the_chunkwise_form():
    """Check [b]: every C gives the same output; only the compute path changes."""
    B, H, L, dk, dv = 1, 1, 40, 4, 7
    q, k, v, dec, _ = _case(3, B, H, L, dk, dv, oracle.DECAY_GATE, with_state=False)
    a = oracle.decay_multipliers(B, H, L, oracle.DECAY_GATE, dec)
    outs = [oracle.chunkwise(q, k, v, a, C)[0] for C in (1, 2, 3, 5, 16, 40, 64)]
    for o in outs[1:]:
        assert oracle.rel_err(o, outs[0]) < 1e-13


def test_state_shape_independent_of_length():
    """Check [c]: the state is d_k x d_v whatever L is (here d_k = 6, d_v = 4)."""
    for L in (0, 1, 13, 100):
        q, k, v, _, _ = _case(4, 1, 1, L, 6, 4, oracle.DECAY_NONE, with_state=False)
        _, S = oracle.recurrent(q, k, v)
        assert S.shape == (1, 1, 6, 4)


# ---------------------------------------------------------------------------
# closed forms and special cases
# ---------------------------------------------------------------------------
def test_final_state_closed_form_blas():
    """No decay, S_0 = 0: S_L = phi(K)^T V, and the last output is phi(q_L)^T phi(K)^T V."""
    q, k, v, _, _ = _case(5, 1, 1, 50, 8, 5, oracle.DECAY_NONE, with_state=False)
    for phi in (oracle.PHI_IDENTITY, oracle.PHI_ELU1):
        out, S = oracle.recurrent(q, k, v, phi)
        fk = oracle.feature_map(k, phi)[0, 0]
        fq = oracle.feature_map(q, phi)[0, 0]
        ref = fk.T @ v[0, 0]
        assert oracle.rel_err(S[0, 0], ref) < 1e-13
        assert oracle.rel_err(out[0, 0, -1], fq[-1] @ ref) < 1e-13


def test_gamma_one_is_the_ungated_form():
    """A per-head gamma of 1 forgets nothing: bit-identical to no decay."""
    q, k, v, _, S0 = _case(6, 1, 2, 20, 4, 4, oracle.DECAY_NONE)
    o1, s1 = oracle.recurrent(q, k, v, state=S0)
    o2, s2 = oracle.recurrent(q, k, v, decay_kind=oracle.DECAY_HEAD, decay=np.ones(2), state=S0)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_constant_gamma_gives_powers():
    """Constant gamma: D[t,s] = gamma^(t-s) (numpy power, no products or logs)."""
    L, gamma = 30, 0.9
    q, k, v, _, _ = _case(7, 1, 1, L, 4, 3, oracle.DECAY_NONE, with_state=False)
    out, _ = oracle.recurrent(q, k, v, decay_kind=oracle.DECAY_HEAD, decay=np.array([gamma]))
    t = np.arange(L)
    D = np.where(t[:, None] >= t[None, :], np.power(gamma, (t[:, None] - t[None, :])), 0.0)
    ref = ((q[0, 0] @ k[0, 0].T) * D) @ v[0, 0]
    assert oracle.rel_err(out[0, 0], ref) < 1e-13


def test_full_forgetting_limit():
    """a_t = 0 for every t: only the current token survives, o_t = (phi(q_t).phi(k_t)) v_t."""
    L = 12
    q, k, v, _, S0 = _case(8, 1, 1, L, 5, 3, oracle.DECAY_NONE)
    for kind, dec in ((oracle.DECAY_LOG, np.full((1, 1, L), -np.inf)),
                      (oracle.DECAY_GATE, np.full((1, 1, L), 800.0))):
        for phi in (oracle.PHI_IDENTITY, oracle.PHI_ELU1):
            out, S = oracle.recurrent(q, k, v, phi, kind, dec, S0)
            fq, fk = oracle.feature_map(q, phi)[0, 0], oracle.feature_map(k, phi)[0, 0]
            ref = np.sum(fq * fk, axis=1)[:, None] * v[0, 0]
            assert oracle.rel_err(out[0, 0], ref) < 1e-13
            assert oracle.rel_err(S[0, 0], np.outer(fk[-1], v[0, 0, -1])) < 1e-13


def test_feature_map_is_torch_elu_plus_one():
    """Read phi out of the oracle (L = 1, S_0 = I, k = 0) and compare with torch's elu + 1."""
    d = 9
    x = np.linspace(-6.0, 4.0, d)
    q = x[None, None, None, :]
    k = np.zeros_like(q)
    v = np.zeros((1, 1, 1, d))
    out, _ = oracle.recurrent(q, k, v, oracle.PHI_ELU1, state=np.eye(d)[None, None])
    ref = (torch.nn.functional.elu(torch.tensor(x, dtype=torch.float64)) + 1.0).numpy()
    assert np.max(np.abs(out[0, 0, 0] - ref)) < 1e-15
    # phi applies to k as well (and not to v): one token with S_0 = 0
    kk = x[None, None, None, :]
    vv = np.arange(1.0, d + 1)[None, None, None, :] - 5.0
    e0 = np.zeros((1, 1, 1, d))
    e0[..., 0] = 1.0  # q = e_0 so that phi(q) = (2, 1, 1, ...)
    out, S = oracle.recurrent(e0, kk, vv, oracle.PHI_ELU1)
    phik = (torch.nn.functional.elu(torch.tensor(x)) + 1.0).numpy()
    assert np.max(np.abs(S[0, 0] - np.outer(phik, vv[0, 0, 0]))) < 1e-14


def test_gate_is_sigmoid_of_minus_g():
    """exp(-softplus(g)) = 1 / (1 + e^g) = sigmoid(-g); read a_t out of the oracle."""
    g = np.array([-30.0, -5.0, -1.0, 0.0, 0.5, 3.0, 20.0, 60.0])
    for gi in g:
        # L = 1, q = e_0, k = 0, S_0 = I: o = a * e_0^T I = a e_0
        q = np.zeros((1, 1, 1, 2))
        q[..., 0] = 1.0
        out, _ = oracle.recurrent(q, np.zeros_like(q), np.zeros((1, 1, 1, 2)),
                                  decay_kind=oracle.DECAY_GATE,
                                  decay=np.array([[[gi]]]), state=np.eye(2)[None, None])
        ref = torch.sigmoid(torch.tensor(-gi, dtype=torch.float64)).item()
        assert abs(out[0, 0, 0, 0] - ref) <= 1e-15 * max(ref, 1e-300) + 1e-300


def test_decay_hits_the_previous_state_only():
    """D[t,t] = 1: the current write is never decayed (one token, S_0 = 0)."""
    q = np.ones((1, 1, 1, 3))
    k = np.ones((1, 1, 1, 3))
    v = np.ones((1, 1, 1, 2))
    out, S = oracle.recurrent(q, k, v, decay_kind=oracle.DECAY_HEAD, decay=np.array([0.5]))
    assert np.array_equal(S[0, 0], np.ones((3, 2)))
    assert np.array_equal(out[0, 0, 0], np.full(2, 3.0))


def test_decode_step_is_one_token_of_the_recurrence():
    """Decode = the recurrence applied one token at a time; 5 steps == one 5-token call."""
    N, H, dk, dv, T = 3, 2, 4, 6, 5
    q, k, v, dec, S0 = _case(9, N, H, T, dk, dv, oracle.DECAY_GATE)
    o_full, S_full = oracle.recurrent(q, k, v, oracle.PHI_ELU1, oracle.DECAY_GATE, dec, S0)
    S = S0
    for t in range(T):
        o, S = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], oracle.PHI_ELU1,
                                  oracle.DECAY_GATE, dec[:, :, t], S)
        assert oracle.rel_err(o, o_full[:, :, t]) < 1e-14
    assert oracle.rel_err(S, S_full) < 1e-14


def test_threads_do_not_change_results():
    q, k, v, dec, S0 = _case(10, 3, 5, 17, 4, 4, oracle.DECAY_LOG)
    o1, s1 = oracle.recurrent(q, k, v, 1, oracle.DECAY_LOG, dec, S0, nthreads=1)
    o2, s2 = oracle.recurrent(q, k, v, 1, oracle.DECAY_LOG, dec, S0, nthreads=7)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


# ---------------------------------------------------------------------------
# the pages' printed numbers and page workloads
# ---------------------------------------------------------------------------
def _page_inputs_13x6():
    g = torch.Generator().manual_seed(0)
    return [torch.randn(13, 6, generator=g).double().numpy() for _ in range(3)]


def test_pages_printed_checks_magnitude():
    """Checks [a]-[c] as printed: L = 13, d = 6, seed 0, C in {1, 4, 7, 13}.

    The page's fp32 run printed max|chunkwise - recurrent| = 3.81e-06 with a
    threshold of 1e-5.  The exact number depends on torch's summation order,
    so the pin is its magnitude: our own chunkwise form evaluated in fp32 on
    the same inputs must sit within the threshold of the fp64 oracle and of
    the same order (1e-7 .. 1e-5); the fp64 forms must agree to ~1e-15.
    """
    gold = json.load(open(os.path.join(GOLDEN, "page_sanity_checks.json")))
    Q, K, V = _page_inputs_13x6()
    q, k, v = Q[None, None], K[None, None], V[None, None]
    ref, S = oracle.recurrent(q, k, v)
    a = np.ones((1, 1, gold["L"]))
    diffs32 = []
    for C in gold["chunk_sizes"]:
        o32, _ = oracle.chunkwise(q.astype(np.float32), k.astype(np.float32),
                                  v.astype(np.float32), a, C, dtype=np.float32)
        diffs32.append(np.max(np.abs(o32 - ref)))
        o64, _ = oracle.chunkwise(q, k, v, a, C)
        assert np.max(np.abs(o64 - ref)) < 1e-13
        assert np.allclose(o64, ref, atol=gold["b_chunk_size_invariance_atol"])
    worst = max(diffs32)
    assert worst < gold["a_threshold"]
    assert gold["a_max_abs_diff_chunkwise_vs_recurrent_fp32"] / 30 < worst < gold["a_threshold"]
    assert [list(S.shape[2:])] == gold["c_state_shapes"]


def test_pages_matrix_form_magnitude():
    """adv13 check 2: the non-causal matrix form phi(Q)(phi(K)^T V) equals the
    non-causal recurrent form to ~1e-7 in fp32 (seq 16, d 32).  Our oracle's
    final state is the non-causal phi(K)^T V; both bracketings in fp32 must
    agree with phi(Q) S_L to the printed order and within atol 1e-5.  The page
    does not say how its inputs were scaled, so both bounds are taken relative
    to max|reference| (a unit-scale output)."""
    gold = json.load(open(os.path.join(GOLDEN, "matrix_form_check.json")))
    n, d = gold["seq"], gold["d"]
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    _, S = oracle.recurrent(q, k, v, oracle.PHI_ELU1)
    fq = oracle.feature_map(q, oracle.PHI_ELU1)[0, 0]
    fk = oracle.feature_map(k, oracle.PHI_ELU1)[0, 0]
    ref = fq @ S[0, 0]
    left = ((fq.astype(np.float32) @ fk.T.astype(np.float32)) @ v[0, 0].astype(np.float32))
    right = fq.astype(np.float32) @ (fk.T.astype(np.float32) @ v[0, 0].astype(np.float32))
    for x in (left, right):
        err = np.max(np.abs(x - ref)) / np.max(np.abs(ref))
        assert err < gold["allclose_atol"]
        assert err < 100 * gold["printed_max_abs_err_order"]


def test_associativity_large():
    """CS336 lecture 4 code 1 demo 1: (Q K^T) V = Q (K^T V) at n = 4096, d = 64, and the
    oracle's final state is K^T V (2 n d^2 flops instead of 2 n^2 d: a ratio n/d = 64)."""
    rng = np.random.default_rng(13)
    n, d = 4096, 64
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    _, S = oracle.recurrent(q[None, None], k[None, None], v[None, None])
    assert oracle.rel_err(S[0, 0], k.T @ v) < 1e-12
    left = (q @ k.T) @ v
    right = q @ S[0, 0]
    assert np.linalg.norm(left - right) / np.linalg.norm(left) < 1e-12
    assert (2 * n * n * d * 2) / (2 * n * d * d * 2) == n / d


def test_small_fp32_workload_inputs_and_forms():
    """The 300 x 16 demo (seed 0, chunk 64): recurrent == parallel == chunked in fp64,
    with the pages' metric max|delta| / max|ref|."""
    q, k, v = W.small_fp32_inputs()
    # the demo's own draw: global manual_seed(0), then randn(300, 16) three times
    torch.manual_seed(0)
    q2, k2, v2 = torch.randn(300, 16), torch.randn(300, 16), torch.randn(300, 16)
    assert torch.equal(q[0, 0], q2) and torch.equal(k[0, 0], k2) and torch.equal(v[0, 0], v2)
    q, k, v = q.double().numpy(), k.double().numpy(), v.double().numpy()
    ref, _ = oracle.recurrent(q, k, v)
    a = np.ones((1, 1, 300))
    op, _ = oracle.parallel(q, k, v, a)
    oc, _ = oracle.chunkwise(q, k, v, a, 64)
    assert oracle.rel_err(op, ref) < 1e-13 and oracle.rel_err(oc, ref) < 1e-13


def test_gated_page_workload():
    """CS336 demo 4: n = 200, d = 16, gamma = sigmoid(k w + 3) per token.  The
    recurrent form must equal the parallel form built from log-space cumsums
    (the page's construction) and our explicit-product parallel form."""
    rng = np.random.default_rng(14)
    n, d = 200, 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    w = rng.standard_normal(d)
    gamma = 1.0 / (1.0 + np.exp(-(k @ w + 3.0)))
    out, _ = oracle.recurrent(q[None, None], k[None, None], v[None, None],
                              decay_kind=oracle.DECAY_LOG, decay=np.log(gamma)[None, None])
    cum = np.cumsum(np.log(gamma))
    causal = np.tril(np.ones((n, n), dtype=bool))
    D = np.where(causal, np.exp(np.where(causal, cum[:, None] - cum[None, :], 0.0)), 0.0)
    ref = ((q @ k.T) * D) @ v
    assert oracle.rel_err(out[0, 0], ref) < 1e-12
    op, _ = oracle.parallel(q[None, None], k[None, None], v[None, None], gamma[None, None])
    assert oracle.rel_err(out, op) < 1e-12


def test_gated_workload_decay_statistics():
    """The gated workload's gate g ~ N(0,1): E[a] = E[sigmoid(-g)] = 1/2 and a
    64-token chunk's log-decay sum lies in tens (the numbers the kernel's
    exp(<=0) design has to survive)."""
    w = W.WORKLOADS["gated_bf16"]
    g = torch.Generator().manual_seed(123)
    x = torch.randn(64 * 4000, generator=g, dtype=torch.float64).numpy()
    a = oracle.decay_multipliers(1, 1, x.size, oracle.DECAY_GATE, x[None, None])[0, 0]
    assert abs(a.mean() - 0.5) < 0.01
    sums = -np.log(a).reshape(-1, w.C).sum(axis=1)
    assert 30 < sums.min() and sums.max() < 80 and abs(sums.mean() - 51.6) < 1.0
    assert math.exp(-sums.max()) > np.finfo(np.float32).tiny


# ---------------------------------------------------------------------------
# the normalised form (tutorial section 2.2, boxed recurrence; z as the extra
# value column of ones, section 6.2)
# ---------------------------------------------------------------------------
def _norm_case(seed, kind, L=23, with_state=True):
    q, k, v, dec, S0 = _case(seed, 1, 2, L, 5, 3, kind, with_state=False)
    rng = np.random.default_rng(seed + 100)
    fk0 = oracle.feature_map(rng.standard_normal((1, 2, 4, 5)), oracle.PHI_ELU1)
    # a consistent initial pair: S_0 = sum of phi(k) v^T, z_0 = sum of phi(k)
    # over 4 earlier tokens, so every denominator stays positive
    v0 = rng.standard_normal((1, 2, 4, 3))
    S0 = np.einsum("bhtk,bhtv->bhkv", fk0, v0) if with_state else None
    z0 = fk0.sum(axis=2) if with_state else None
    return q, k, v, dec, S0, z0


@pytest.mark.parametrize("kind", [oracle.DECAY_NONE, oracle.DECAY_HEAD, oracle.DECAY_LOG,
                                  oracle.DECAY_GATE])
def test_normalised_recurrent_equals_parallel_and_chunkwise(kind):
    q, k, v, dec, S0, z0 = _norm_case(11 + kind, kind)
    a = oracle.decay_multipliers(1, 2, 23, kind, dec)
    o, S, Z = oracle.recurrent(q, k, v, oracle.PHI_ELU1, kind, dec, S0, normalize=True,
                               norm_state=z0)
    op, Sp = oracle.parallel(q, k, v, a, oracle.PHI_ELU1, S0, normalize=True, norm_state=z0)
    assert np.abs(o - op).max() < 1e-12 * max(1.0, np.abs(op).max())
    for C in (1, 4, 7, 23):
        oc, Sc, Zc = oracle.chunkwise(q, k, v, a, C, oracle.PHI_ELU1, S0, normalize=True,
                                      norm_state=z0)
        assert np.abs(o - oc).max() < 1e-12 * max(1.0, np.abs(o).max())
        assert np.abs(Z - Zc).max() < 1e-12 * max(1.0, np.abs(Z).max())
    # the normaliser is the un-normalised output for v = 1 (z is S's column of ones)
    ones = np.ones((1, 2, 23, 1))
    den, zS = oracle.recurrent(q, k, ones, oracle.PHI_ELU1, kind, dec, z0[..., None])
    num, _ = oracle.recurrent(q, k, v, oracle.PHI_ELU1, kind, dec, S0)
    assert np.abs(o - num / den).max() < 1e-12 * max(1.0, np.abs(o).max())
    assert np.abs(Z - zS[..., 0]).max() < 1e-12 * np.abs(Z).max()


def test_normalised_first_token_returns_its_value():
    # z_0 = 0, S_0 = 0: o_0 = (phi(q).phi(k) v_0) / (phi(q).phi(k)) = v_0
    q, k, v, dec, _, _ = _norm_case(5, oracle.DECAY_GATE, with_state=False)
    o, _, _ = oracle.recurrent(q, k, v, oracle.PHI_ELU1, oracle.DECAY_GATE, dec, normalize=True)
    assert np.allclose(o[:, :, 0], v[:, :, 0], rtol=1e-14, atol=1e-14)


def test_normalised_output_is_a_convex_combination_of_values():
    # phi = elu + 1 > 0 and no decay: o_t = sum_s w_ts v_s with w_ts > 0, sum_s w_ts = 1
    q, k, v, _, _, _ = _norm_case(6, oracle.DECAY_NONE, L=40, with_state=False)
    o, _, _ = oracle.recurrent(q, k, v, oracle.PHI_ELU1, oracle.DECAY_NONE, normalize=True)
    lo = np.minimum.accumulate(v, axis=2)
    hi = np.maximum.accumulate(v, axis=2)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


@pytest.mark.parametrize("kind", [oracle.DECAY_HEAD, oracle.DECAY_GATE])
def test_normalised_constant_values_pass_through(kind):
    # v_t = c for every t (and S_0 = z_0 c^T): every output is exactly c
    q, k, _, dec, _, z0 = _norm_case(7, kind)
    c = np.array([0.5, -2.0, 3.0])
    v = np.broadcast_to(c, (1, 2, 23, 3)).copy()
    S0 = z0[..., None] * c
    o, _, _ = oracle.recurrent(q, k, v, oracle.PHI_ELU1, kind, dec, S0, normalize=True,
                               norm_state=z0)
    assert np.allclose(o, c, rtol=1e-12, atol=1e-12)


def test_normalised_decode_step_is_one_token():
    q, k, v, dec, S0, z0 = _norm_case(8, oracle.DECAY_LOG, L=1)
    o, S, Z = oracle.recurrent(q, k, v, oracle.PHI_ELU1, oracle.DECAY_LOG, dec, S0,
                               normalize=True, norm_state=z0)
    od, Sd, Zd = oracle.decode_step(q[:, :, 0], k[:, :, 0], v[:, :, 0], oracle.PHI_ELU1,
                                    oracle.DECAY_LOG, dec[:, :, 0], S0, normalize=True,
                                    norm_state=z0)
    assert np.array_equal(o[:, :, 0], od) and np.array_equal(S, Sd) and np.array_equal(Z, Zd)


# ---------------------------------------------------------------------------
# the per-channel (GLA) gate, tutorial section 2.4: S_t = diag(alpha_t) S_{t-1} + k v^T
# ---------------------------------------------------------------------------
def _channel_case(seed, L=19, dk=5, dv=3, strength=0.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 2, L, dk))
    k = rng.standard_normal((1, 2, L, dk))
    v = rng.standard_normal((1, 2, L, dv))
    la = -np.abs(rng.standard_normal((1, 2, L, dk))) * strength
    S0 = rng.standard_normal((1, 2, dk, dv))
    return q, k, v, la, S0


@pytest.mark.parametrize("phi", [oracle.PHI_IDENTITY, oracle.PHI_ELU1])
def test_channel_gate_recurrent_equals_parallel_and_chunkwise(phi):
    q, k, v, la, S0 = _channel_case(40 + phi)
    o, S = oracle.recurrent(q, k, v, phi, oracle.DECAY_CHANNEL, la, S0)
    op, Sp = oracle.parallel_channel(q, k, v, np.exp(la), phi, S0)
    assert oracle.rel_err(o, op) < 1e-13 and oracle.rel_err(S, Sp) < 1e-13
    for C in (1, 4, 7, 19):
        oc, Sc = oracle.chunkwise_channel(q, k, v, la, C, phi, S0)
        assert oracle.rel_err(o, oc) < 1e-13 and oracle.rel_err(S, Sc) < 1e-13


def test_channel_gate_with_equal_channels_is_the_scalar_gate():
    # alpha_t the same in every channel: the scalar log-decay recurrence
    q, k, v, la, S0 = _channel_case(43)
    la_tok = la[..., 0]
    la_all = np.repeat(la_tok[..., None], q.shape[-1], axis=-1)
    o, S = oracle.recurrent(q, k, v, oracle.PHI_IDENTITY, oracle.DECAY_CHANNEL, la_all, S0)
    os_, Ss = oracle.recurrent(q, k, v, oracle.PHI_IDENTITY, oracle.DECAY_LOG, la_tok, S0)
    assert oracle.rel_err(o, os_) < 1e-14 and oracle.rel_err(S, Ss) < 1e-14


def test_channel_gate_exact_rational_sum():
    # integer q, k, v and dyadic per-channel gates: the definition in rationals
    rng = np.random.default_rng(44)
    L, dk, dv = 6, 3, 2
    q = rng.integers(-3, 4, (L, dk))
    k = rng.integers(-3, 4, (L, dk))
    v = rng.integers(-3, 4, (L, dv))
    a = rng.choice([Fraction(1, 2), Fraction(3, 4), Fraction(1)], size=(L, dk))
    S0 = rng.integers(-2, 3, (dk, dv))
    S = [[Fraction(int(S0[i][j])) for j in range(dv)] for i in range(dk)]
    ref = []
    for t in range(L):
        for i in range(dk):
            for j in range(dv):
                S[i][j] = a[t][i] * S[i][j] + int(k[t][i]) * int(v[t][j])
        ref.append([sum(int(q[t][i]) * S[i][j] for i in range(dk)) for j in range(dv)])
    la = np.log(np.array([[float(x) for x in row] for row in a]))
    o, Sg = oracle.recurrent(q[None, None], k[None, None], v[None, None], oracle.PHI_IDENTITY,
                             oracle.DECAY_CHANNEL, la[None, None], S0[None, None].astype(float))
    assert np.max(np.abs(o[0, 0] - np.array(ref, dtype=float))) < 1e-12
    assert np.max(np.abs(Sg[0, 0] - np.array([[float(x) for x in r] for r in S]))) < 1e-12


def test_channel_gate_decays_rows_of_the_state():
    # one channel fully forgotten each step (log a = -inf): that row of S keeps
    # only the newest write, the other rows accumulate
    q, k, v, la, S0 = _channel_case(45, L=5, dk=3, dv=2)
    la[:] = 0.0
    la[..., 1] = -np.inf
    _, S = oracle.recurrent(q, k, v, oracle.PHI_IDENTITY, oracle.DECAY_CHANNEL, la, S0)
    newest = k[:, :, -1, 1, None] * v[:, :, -1, :]
    assert np.allclose(S[:, :, 1, :], newest, rtol=1e-14, atol=1e-14)
    acc = S0[:, :, 0, :] + np.einsum("bht,bhtv->bhv", k[..., 0], v)
    assert np.allclose(S[:, :, 0, :], acc, rtol=1e-13, atol=1e-13)


def test_channel_gate_decode_step_is_one_token():
    q, k, v, la, S0 = _channel_case(46, L=1)
    o, S = oracle.recurrent(q, k, v, oracle.PHI_ELU1, oracle.DECAY_CHANNEL, la, S0)
    od, Sd = oracle.decode_step(q[:, :, 0], k[:, :, 0], v[:, :, 0], oracle.PHI_ELU1,
                                oracle.DECAY_CHANNEL, la[:, :, 0], S0)
    assert np.array_equal(o[:, :, 0], od) and np.array_equal(S, Sd)


# ---------------------------------------------------------------------------
# the normalised form under the per-channel gate (tutorial section 2.2 boxed
# recurrence with section 2.4's diagonal gate: z decays per channel like each
# row of S, since z is S's extra value column of ones, section 6.2)
# ---------------------------------------------------------------------------
def _channel_norm_case(seed, L=19, dk=5, dv=3):
    q, k, v, la, _ = _channel_case(seed, L, dk, dv)
    rng = np.random.default_rng(seed + 500)
    # a consistent positive initial pair, as after 4 earlier tokens
    fk0 = oracle.feature_map(rng.standard_normal((1, 2, 4, dk)), oracle.PHI_ELU1)
    v0 = rng.standard_normal((1, 2, 4, dv))
    return q, k, v, la, np.einsum("bhtk,bhtv->bhkv", fk0, v0), fk0.sum(axis=2)


def test_channel_gate_normalised_recurrent_equals_parallel_and_chunkwise():
    q, k, v, la, S0, z0 = _channel_norm_case(60)
    o, S, Z = oracle.recurrent(q, k, v, oracle.PHI_ELU1, oracle.DECAY_CHANNEL, la, S0,
                               normalize=True, norm_state=z0)
    op, Sp = oracle.parallel_channel(q, k, v, np.exp(la), oracle.PHI_ELU1, S0, normalize=True,
                                     norm_state=z0)
    assert oracle.rel_err(o, op) < 1e-13 and oracle.rel_err(S, Sp) < 1e-13
    for C in (1, 4, 7, 19):
        oc, Sc, Zc = oracle.chunkwise_channel(q, k, v, la, C, oracle.PHI_ELU1, S0,
                                              normalize=True, norm_state=z0)
        assert oracle.rel_err(o, oc) < 1e-13 and oracle.rel_err(S, Sc) < 1e-13
        assert oracle.rel_err(Z, Zc) < 1e-13


def test_channel_gate_normalised_with_equal_channels_is_the_scalar_gate():
    # alpha_t equal in every channel: the normalised scalar log-decay recurrence
    q, k, v, la, S0, z0 = _channel_norm_case(61)
    la_tok = la[..., 0]
    la_all = np.repeat(la_tok[..., None], q.shape[-1], axis=-1)
    o, S, Z = oracle.recurrent(q, k, v, oracle.PHI_ELU1, oracle.DECAY_CHANNEL, la_all, S0,
                               normalize=True, norm_state=z0)
    os_, Ss, Zs = oracle.recurrent(q, k, v, oracle.PHI_ELU1, oracle.DECAY_LOG, la_tok, S0,
                                   normalize=True, norm_state=z0)
    assert oracle.rel_err(o, os_) < 1e-14 and oracle.rel_err(Z, Zs) < 1e-14


def test_channel_gate_normalised_z_is_the_state_for_unit_values():
    # z_t is exactly the un-normalised state's column for v = 1, decayed per channel,
    # and the output is the un-normalised output divided by that column's read-out
    q, k, v, la, S0, z0 = _channel_norm_case(62)
    o, _, Z = oracle.recurrent(q, k, v, oracle.PHI_ELU1, oracle.DECAY_CHANNEL, la, S0,
                               normalize=True, norm_state=z0)
    ones = np.ones(v.shape[:-1] + (1,))
    den, zS = oracle.recurrent(q, k, ones, oracle.PHI_ELU1, oracle.DECAY_CHANNEL, la,
                               z0[..., None])
    num, _ = oracle.recurrent(q, k, v, oracle.PHI_ELU1, oracle.DECAY_CHANNEL, la, S0)
    assert oracle.rel_err(Z, zS[..., 0]) < 1e-14
    assert oracle.rel_err(o, num / den) < 1e-13


def test_channel_gate_normalised_forgotten_channel():
    # a channel with log a = -inf forgets z's entry every step: z_d = phi(k_t)_d of the newest
    # token; a channel with log a = 0 accumulates: z_d = z0_d + sum_t phi(k_t)_d
    q, k, v, la, S0, z0 = _channel_norm_case(63, L=6, dk=3, dv=2)
    la[:] = 0.0
    la[..., 2] = -np.inf
    _, _, Z = oracle.recurrent(q, k, v, oracle.PHI_ELU1, oracle.DECAY_CHANNEL, la, S0,
                               normalize=True, norm_state=z0)
    fk = oracle.feature_map(k, oracle.PHI_ELU1)
    assert np.allclose(Z[..., 2], fk[:, :, -1, 2], rtol=1e-14, atol=0)
    assert np.allclose(Z[..., 0], z0[..., 0] + fk[..., 0].sum(axis=2), rtol=1e-13, atol=0)
