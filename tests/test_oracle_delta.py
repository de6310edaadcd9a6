"""Pins of the oracle's delta rule (DeltaNet; Gated DeltaNet with a scalar
decay) against what the pages and the mathematics fix.  CPU only.

The oracle (`oracle.delta_recurrent`, C) is checked against:
  * the pages' own form: a value-by-key state with explicit (I - beta k k^T)
    factors ("Linear / Sparse Attention", delta_rule_recurrent; tutorial
    Q17 for the gate), computed in numpy in the other orientation;
  * the chunkwise WY / UT form for several chunk sizes;
  * the printed sanity check [e] of "Linear / Sparse Attention" on its own
    seeded inputs (tests/golden/page_delta_checks.json);
  * closed forms: the just-written key reads back its value (beta = 1, unit
    keys), beta = 0 leaves pure decay, orthonormal keys reduce to additive
    linear attention (check [e]);
  * exact rational arithmetic on integer inputs.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_delta_checks.json")


def _inputs(seed, B=2, H=3, L=29, dk=7, dv=5, unit=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    if unit:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, L, dv))
    beta = rng.uniform(0.05, 1.0, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.5
    decays = {
        oracle.DECAY_NONE: None,
        oracle.DECAY_HEAD: rng.uniform(0.6, 1.0, H),
        oracle.DECAY_LOG: -np.abs(rng.standard_normal((B, H, L))) * 0.3,
        oracle.DECAY_GATE: rng.standard_normal((B, H, L)),
    }
    return q, k, v, beta, S0, decays


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
def test_delta_recurrent_equals_the_pages_explicit_form(kind):
    q, k, v, beta, S0, decays = _inputs(1)
    B, H, L, _ = q.shape
    o, S = oracle.delta_recurrent(q, k, v, beta, kind, decays[kind], S0)
    a = oracle.decay_multipliers(B, H, L, kind, decays[kind])
    oe, Se = oracle.delta_explicit(q, k, v, beta, a, S0)
    assert oracle.rel_err(o, oe) < 1e-12 and oracle.rel_err(S, Se) < 1e-12


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
def test_delta_chunkwise_equals_recurrent_for_every_chunk_size(kind):
    q, k, v, beta, S0, decays = _inputs(2)
    B, H, L, _ = q.shape
    o, S = oracle.delta_recurrent(q, k, v, beta, kind, decays[kind], S0)
    la = np.log(oracle.decay_multipliers(B, H, L, kind, decays[kind]))
    for C in (1, 4, 7, 16, L):
        oc, Sc = oracle.delta_chunkwise(q, k, v, beta, la, C, S0)
        assert oracle.rel_err(oc, o) < 1e-12 and oracle.rel_err(Sc, S) < 1e-12, C


def _page_inputs():
    torch.manual_seed(0)
    L, d = 13, 6
    _q, _k, V = torch.randn(L, d), torch.randn(L, d), torch.randn(L, d)
    Kn = F.normalize(torch.randn(L, d), dim=-1)
    qm, _ = torch.linalg.qr(torch.randn(d, d))
    Ko = qm.t()[:d]
    Vo = torch.randn(d, d)
    f = lambda x: x.double().numpy()[None, None]  # noqa: E731
    return f(Kn), f(V), f(Ko), f(Vo)


def test_page_check_e_printed_values():
    """Check [e] on the script's own inputs: non-orthogonal unit keys with
    beta = 1 move the final state away from the additive one by the printed
    Frobenius norm; orthonormal keys leave it (within fp32 keys) unchanged."""
    g = json.load(open(GOLDEN))
    Kn, V, Ko, Vo = _page_inputs()
    L, d = g["L"], g["d"]
    _, Sd = oracle.delta_recurrent(np.zeros((1, 1, L, d)), Kn, V, np.ones((1, 1, L)))
    _, Sa = oracle.recurrent(np.zeros((1, 1, L, d)), Kn, V)
    diff = float(np.linalg.norm(Sd - Sa))
    assert abs(diff - g["e_nonorthogonal_frobenius_diff"]) < 0.5e-3
    assert diff > g["e_nonorthogonal_threshold"]
    _, Sdo = oracle.delta_recurrent(np.zeros((1, 1, d, d)), Ko, Vo, np.ones((1, 1, d)))
    _, Sao = oracle.recurrent(np.zeros((1, 1, d, d)), Ko, Vo)
    # the keys are orthonormal only to fp32 precision: the residual stays below
    # what the script printed for its fp32 run
    assert np.abs(Sdo - Sao).max() <= g["e_orthonormal_max_abs_diff_fp32"]


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
def test_orthonormal_keys_with_unit_beta_are_additive(kind):
    """Check [e]'s sufficient condition in fp64, decayed too: from S_0 = 0 the
    erase term sees only earlier, orthogonal keys, so it vanishes."""
    rng = np.random.default_rng(3)
    d, B, H = 8, 1, 2
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = np.broadcast_to(Qm.T, (B, H, d, d)).copy()
    q = rng.standard_normal((B, H, d, d))
    v = rng.standard_normal((B, H, d, 3))
    _, _, _, _, _, decays = _inputs(3, B=B, H=H, L=d)
    dec = decays[kind]
    o, S = oracle.delta_recurrent(q, k, v, np.ones((B, H, d)), kind, dec)
    oa, Sa = oracle.recurrent(q, k, v, 0, kind, dec)
    assert oracle.rel_err(o, oa) < 1e-13 and oracle.rel_err(S, Sa) < 1e-13


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
def test_written_key_reads_back_its_value(kind):
    """beta = 1 and a unit key: the step stores v_t under k_t exactly
    (S_t^T k_t = v_t, one step of the online least-squares view, tutorial Q15),
    whatever the decayed previous state held."""
    q, k, v, beta, S0, decays = _inputs(4)
    o, _ = oracle.delta_recurrent(k, k, v, np.ones_like(beta), kind, decays[kind], S0)
    assert np.max(np.abs(o - v)) < 1e-12


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
def test_zero_beta_is_pure_decay(kind):
    q, k, v, beta, S0, decays = _inputs(5)
    B, H, L, _ = q.shape
    o, S = oracle.delta_recurrent(q, k, v, np.zeros_like(beta), kind, decays[kind], S0)
    a = np.cumprod(oracle.decay_multipliers(B, H, L, kind, decays[kind]), axis=-1)
    ref = a[..., None] * np.einsum("bhtd,bhde->bhte", q, S0)
    assert oracle.rel_err(o, ref) < 1e-13
    assert oracle.rel_err(S, a[..., -1, None, None] * S0) < 1e-13


def test_exact_rational_sums():
    """Integer q, k, v, S_0 and beta = 1/4: the recurrence is a polynomial in
    the inputs, so exact Fractions give the true values."""
    rng = np.random.default_rng(6)
    L, dk, dv = 6, 3, 2
    q = rng.integers(-2, 3, (L, dk))
    k = rng.integers(-1, 2, (L, dk))
    v = rng.integers(-3, 4, (L, dv))
    S0 = rng.integers(-2, 3, (dk, dv))
    gamma = Fraction(3, 4)
    beta = Fraction(1, 4)
    S = [[Fraction(int(S0[i, j])) for j in range(dv)] for i in range(dk)]
    want = []
    for t in range(L):
        r = [sum(Fraction(int(k[t, i])) * S[i][j] for i in range(dk)) for j in range(dv)]
        S = [[gamma * (S[i][j] - beta * int(k[t, i]) * r[j]) + beta * int(k[t, i]) * int(v[t, j])
              for j in range(dv)] for i in range(dk)]
        want.append([sum(int(q[t, i]) * S[i][j] for i in range(dk)) for j in range(dv)])
    o, Sl = oracle.delta_recurrent(q[None, None], k[None, None], v[None, None],
                                   np.full((1, 1, L), 0.25), oracle.DECAY_HEAD,
                                   np.array([0.75]), S0[None, None].astype(float))
    assert np.max(np.abs(o[0, 0] - np.array(want, dtype=float))) < 1e-12
    assert np.max(np.abs(Sl[0, 0] - np.array(S, dtype=float))) < 1e-12


def test_delta_decode_step_is_one_token():
    q, k, v, beta, S0, decays = _inputs(7, L=5)
    o, S = oracle.delta_recurrent(q, k, v, beta, oracle.DECAY_GATE, decays[3], S0)
    Sd = S0.copy()
    for t in range(5):
        ot, Sd = oracle.delta_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], beta[:, :, t],
                                          oracle.DECAY_GATE, decays[3][:, :, t], Sd)
        assert np.max(np.abs(ot - o[:, :, t])) < 1e-13
    assert np.max(np.abs(Sd - S)) < 1e-13


def test_delta_threads_do_not_change_results():
    q, k, v, beta, S0, decays = _inputs(8)
    o1, S1 = oracle.delta_recurrent(q, k, v, beta, 3, decays[3], S0, nthreads=1)
    o4, S4 = oracle.delta_recurrent(q, k, v, beta, 3, decays[3], S0, nthreads=4)
    assert np.array_equal(o1, o4) and np.array_equal(S1, S4)
