"""Plant plausible mistakes in copies of the oracle and check that the pins catch each one.

Every mutant is the oracle's C source with one small textual change (a
dropped term, a wrong sign, index or operand, a transposed state), compiled
with gcc into a temporary directory.  A compact battery of the pins from
test_oracle_pins.py runs against each copy; each mutant must fail at least
one check, and the unmodified source must pass them all.  Nothing here runs
on a GPU.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "la_oracle.c")

MUTANTS = {
    "decay_hits_current_write": ("ai * S[(size_t)i * dv + j] + fk[i] * vt[j]",
                                 "ai * (S[(size_t)i * dv + j] + fk[i] * vt[j])"),
    "query_written_instead_of_key": ("+ fk[i] * vt[j]", "+ fq[i] * vt[j]"),
    "elu_plus_one_garbled": ("return x > 0.0 ? x + 1.0 : exp(x);",
                             "return x > 0.0 ? x + 1.0 : exp(x) + 1.0;"),
    "gate_sign_flipped": ("return exp(-oracle_softplus(dh[t]));",
                          "return exp(-oracle_softplus(-dh[t]));"),
    "softplus_term_dropped": ("log1p(exp(-fabs(g)))", "0.0 * log1p(exp(-fabs(g)))"),
    "read_before_write": ("acc += fq[i] * S[(size_t)i * dv + j];",
                          "acc += fq[i] * (S[(size_t)i * dv + j] - fk[i] * vt[j]);"),
    "state_read_transposed": ("acc += fq[i] * S[(size_t)i * dv + j];",
                              "acc += fq[i] * S[(size_t)j * dk + i];"),
    "head_decay_of_head_zero": ("dh = j->decay + h;", "dh = j->decay;"),
    "token_decay_off_by_one": ("case ORACLE_DECAY_LOG: return exp(dh[t]);",
                               "case ORACLE_DECAY_LOG: return exp(dh[t > 0 ? t - 1 : 0]);"),
    "feature_map_on_values": ("+ fk[i] * vt[j];", "+ fk[i] * oracle_phi(phi, vt[j]);"),
    "normaliser_not_decayed": ("z[i] = ai * z[i] + fk[i];", "z[i] = z[i] + fk[i];"),
    "normaliser_of_queries": ("z[i] = ai * z[i] + fk[i];", "z[i] = ai * z[i] + fq[i];"),
    "denominator_with_keys": ("den += fq[i] * z[i];", "den += fk[i] * z[i];"),
    "channel_gate_reversed": ("? exp(dh[(size_t)t * dk + i]) : a;",
                              "? exp(dh[(size_t)t * dk + (dk - 1 - i)]) : a;"),
    "normaliser_channel_gate_scalar": (
        "? exp(dh[(size_t)t * dk + i]) : a;\n        z[i] = ai * z[i] + fk[i];",
        "? a : a;\n        z[i] = ai * z[i] + fk[i];"),
    "channel_gate_of_previous_token": ("? exp(dh[(size_t)t * dk + i]) : a;",
                                       "? exp(dh[(size_t)(t > 0 ? t - 1 : 0) * dk + i]) : a;"),
    # the delta rule
    "delta_erase_along_query": ("acc += kt[i] * S[(size_t)i * dv + j];",
                                "acc += qt[i] * S[(size_t)i * dv + j];"),
    "delta_beta_missing_on_erase": ("a * (S[(size_t)i * dv + j] - bt * kt[i] * r[j])",
                                    "a * (S[(size_t)i * dv + j] - kt[i] * r[j])"),
    "delta_write_decayed": ("+ bt * kt[i] * vt[j];", "+ a * bt * kt[i] * vt[j];"),
    "delta_erase_not_decayed": ("a * (S[(size_t)i * dv + j] - bt * kt[i] * r[j])",
                                "a * S[(size_t)i * dv + j] - bt * kt[i] * r[j]"),
}


def _compile(src_text: str, out_dir: str, name: str) -> str:
    c = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", so, c, "-lm",
                    "-lpthread"], check=True, capture_output=True)
    return so


def _battery(lib):
    """Return the names of the failed checks (empty list = all pass)."""
    failed = []
    rng = np.random.default_rng(99)
    B, H, L, dk, dv = 2, 3, 11, 5, 3
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    v = rng.standard_normal((B, H, L, dv))
    S0 = rng.standard_normal((B, H, dk, dv))
    decays = {
        oracle.DECAY_NONE: None,
        oracle.DECAY_HEAD: rng.uniform(0.5, 1.0, H),
        oracle.DECAY_LOG: -np.abs(rng.standard_normal((B, H, L))) * 0.5,
        oracle.DECAY_GATE: rng.standard_normal((B, H, L)),
    }
    # recurrent == parallel (explicit products) for every variant
    for phi in (oracle.PHI_IDENTITY, oracle.PHI_ELU1):
        for kind, dec in decays.items():
            o, S = oracle.recurrent(q, k, v, phi, kind, dec, S0, lib_path=lib)
            a = oracle.decay_multipliers(B, H, L, kind, dec)
            op, Sp = oracle.parallel(q, k, v, a, phi, S0)
            if oracle.rel_err(o, op) > 1e-12 or oracle.rel_err(S, Sp) > 1e-12:
                failed.append(f"parallel phi={phi} kind={kind}")
    # the normalised form: recurrent == parallel (explicit products, masked row sums)
    for kind, dec in decays.items():
        o, S, Z = oracle.recurrent(q, k, v, oracle.PHI_ELU1, kind, dec, normalize=True,
                                   lib_path=lib)
        a = oracle.decay_multipliers(B, H, L, kind, dec)
        op, _ = oracle.parallel(q, k, v, a, oracle.PHI_ELU1, normalize=True)
        if oracle.rel_err(o, op) > 1e-12:
            failed.append(f"normalised parallel kind={kind}")
    # the per-channel gate: recurrent == parallel with explicit per-channel products
    la = -np.abs(rng.standard_normal((B, H, L, dk))) * 0.5
    for phi in (oracle.PHI_IDENTITY, oracle.PHI_ELU1):
        o, S = oracle.recurrent(q, k, v, phi, oracle.DECAY_CHANNEL, la, S0, lib_path=lib)
        op, Sp = oracle.parallel_channel(q, k, v, np.exp(la), phi, S0)
        if oracle.rel_err(o, op) > 1e-12 or oracle.rel_err(S, Sp) > 1e-12:
            failed.append(f"channel gate phi={phi}")
    # the normalised form under the per-channel gate: recurrent == parallel (explicit products)
    z0 = np.abs(rng.standard_normal((B, H, dk))) + 0.5
    o, S, Z = oracle.recurrent(q, k, v, oracle.PHI_ELU1, oracle.DECAY_CHANNEL, la, None,
                               normalize=True, norm_state=z0, lib_path=lib)
    op, _ = oracle.parallel_channel(q, k, v, np.exp(la), oracle.PHI_ELU1, normalize=True,
                                    norm_state=z0)
    if oracle.rel_err(o, op) > 1e-12:
        failed.append("normalised channel gate")
    # the delta rule: the C recurrence == the pages' explicit (I - beta k k^T) form
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    beta = rng.uniform(0.1, 1.0, (B, H, L))
    for kind, dec in decays.items():
        o, S = oracle.delta_recurrent(q, kn, v, beta, kind, dec, S0, lib_path=lib)
        a = oracle.decay_multipliers(B, H, L, kind, dec)
        oe, Se = oracle.delta_explicit(q, kn, v, beta, a, S0)
        if oracle.rel_err(o, oe) > 1e-12 or oracle.rel_err(S, Se) > 1e-12:
            failed.append(f"delta explicit kind={kind}")
    # phi read out against torch's elu + 1
    x = np.linspace(-4.0, 3.0, 6)
    o, _ = oracle.recurrent(x[None, None, None], np.zeros((1, 1, 1, 6)), np.zeros((1, 1, 1, 6)),
                            oracle.PHI_ELU1, state=np.eye(6)[None, None], lib_path=lib)
    ref = (torch.nn.functional.elu(torch.tensor(x)) + 1.0).numpy()
    if np.max(np.abs(o[0, 0, 0] - ref)) > 1e-14:
        failed.append("elu")
    # gate read out against torch.sigmoid(-g)
    for g in (-3.0, 0.7, 5.0):
        qq = np.zeros((1, 1, 1, 2))
        qq[..., 0] = 1.0
        o, _ = oracle.recurrent(qq, np.zeros_like(qq), np.zeros((1, 1, 1, 2)),
                                decay_kind=oracle.DECAY_GATE, decay=np.array([[[g]]]),
                                state=np.eye(2)[None, None], lib_path=lib)
        if abs(o[0, 0, 0, 0] - torch.sigmoid(torch.tensor(-g, dtype=torch.float64)).item()) > 1e-15:
            failed.append(f"gate g={g}")
    return failed


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_unmodified_oracle_passes_the_battery(workdir):
    lib = _compile(open(SRC).read(), workdir, "original")
    assert _battery(lib) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(workdir, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found in la_oracle.c"
    lib = _compile(src.replace(old, new, 1), workdir, name)
    assert _battery(lib), f"mutant {name} passed every pin"
