"""Pins of the Muir gate-prologue oracle (CPU only).

Page: "Muir: Linear Attention with Sensitivity-Allocated Gating and
Matched-Filter Readout", §2.1 (gate parameterisation, eq.(1)) and §4.1
(eq.(8)-(9) and the gate list after eq.(9)).
"""
import math

import numpy as np
import pytest

import oracle
from oracle import muir as MU
from synth import muir_inputs


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _one(x):
    return np.full((1, 1, 1, 1), x, dtype=np.float64)


def test_decay_closed_forms():
    """softplus(0) = ln 2, so z_f = 0 gives alpha = 2^(-exp(a_log)): 1/2 at a_log = 0
    and 1/8 at a_log = ln 3; z_f -> -inf gives alpha -> 1 (no decay)."""
    z0 = _one(0.0)
    a, _, _, _ = oracle.muir_gates(z0, z0, z0, [0.0])
    assert abs(a.item() - 0.5) < 1e-16
    a, _, _, _ = oracle.muir_gates(z0, z0, z0, [math.log(3.0)])
    assert abs(a.item() - 0.125) < 1e-16
    a, _, _, _ = oracle.muir_gates(_one(-800.0), z0, z0, [0.0])
    assert a.item() == 1.0
    # large logits: softplus(z) = z + log1p(e^-z), so log alpha = -e^a (z + e^-z) to first order
    z = 40.0
    a, _, _, _ = oracle.muir_gates(_one(z), z0, z0, [-2.0])
    assert abs(math.log(a.item()) + math.exp(-2.0) * (z + math.exp(-z))) < 1e-12


def test_gate_ranges_and_centres():
    """b = 2 sigmoid in (0, 2) centred at 1, w = sigmoid in (0, 1) centred at 1/2,
    alpha in (0, 1]; sigmoid(-z) = 1 - sigmoid(z)."""
    rng = np.random.default_rng(0)
    z = rng.standard_normal((2, 3, 50, 8)) * 6
    a, b, w, g = oracle.muir_gates(z, z, z, rng.standard_normal(3), z, np.ones((3, 8)))
    assert np.all((a > 0) & (a <= 1)) and np.all((b > 0) & (b < 2)) and np.all((w > 0) & (w < 1))
    _, b0, w0, g0 = oracle.muir_gates(_one(0.0), _one(0.0), _one(0.0), [0.0], _one(0.0), np.ones((1, 1)))
    assert b0.item() == 1.0 and w0.item() == 0.5 and g0.item() == 1.0
    assert np.allclose(MU.sigmoid(-z), 1.0 - MU.sigmoid(z), rtol=0, atol=1e-15)


def test_erase_eigenvalue_in_open_unit_interval():
    """With unit keys and b in (0, 2), the erase factor's eigenvalue along k,
    1 - <k, b*k>, lies in (-1, 1) (§2.1, after eq.(1))."""
    rng = np.random.default_rng(1)
    k = rng.standard_normal((1, 2, 200, 16))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    _, b, _, _ = oracle.muir_gates(k, rng.standard_normal(k.shape) * 5, k, [0.0, 0.0])
    lam = 1.0 - np.sum(k * b * k, axis=-1)
    assert np.all(np.abs(lam) < 1.0)


def test_initialisation_gain_is_one_and_reduces_to_gdn2():
    """At initialisation (z_q = 0, gamma_stat = 1) gamma = 1 and the Muir
    recurrence is GDN-2 on the same gates."""
    d = muir_inputs(2, 3, 40, 6, 5, seed=3, dtype="f32", with_gamma=False, s0_std=0.3)
    o1, S1 = oracle.muir_recurrent(d["q"], d["k"], d["v"], d["z_f"], d["z_b"], d["z_w"], d["a_log"],
                                   None, None, S0=d["S0"])
    a, b, w, g = oracle.muir_gates(d["z_f"], d["z_b"], d["z_w"], d["a_log"])
    assert np.all(g == 1.0)
    o2, S2 = oracle.gdn2_recurrent(d["q"], d["k"], d["v"], a, b, w, S0=d["S0"])
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_gain_acts_on_the_readout_only():
    """gamma scales q at readout (eq.(8)): the state does not depend on z_q or
    gamma_stat, and o is linear in gamma_stat. A gain applied to k instead
    changes the state."""
    d = muir_inputs(1, 2, 30, 6, 4, seed=4, dtype="f32", s0_std=0.2)
    args = (d["q"], d["k"], d["v"], d["z_f"], d["z_b"], d["z_w"], d["a_log"])
    o1, S1 = oracle.muir_recurrent(*args, d["z_q"], d["gamma_stat"], S0=d["S0"])
    o2, S2 = oracle.muir_recurrent(*args, -d["z_q"], 3.0 * d["gamma_stat"], S0=d["S0"])
    assert np.array_equal(S1, S2)
    o3, _ = oracle.muir_recurrent(*args, d["z_q"], 3.0 * d["gamma_stat"], S0=d["S0"])
    assert _rel(o3, 3.0 * o1) < 1e-14
    # planted mistake: the gain on the key
    a, b, w, g = oracle.muir_gates(d["z_f"], d["z_b"], d["z_w"], d["a_log"], d["z_q"], d["gamma_stat"])
    _, S_bad = oracle.gdn2_recurrent(d["q"], g * d["k"], d["v"], a, b, w, S0=d["S0"])
    assert _rel(S_bad, S1) > 1e-2


def test_hand_worked_single_step():
    """One token, d_k = d_v = 1, S0 = s: alpha = 2^-(e^0) = 1/2 (z_f = 0),
    b = 2 sigmoid(0) = 1, w = sigmoid(0) = 1/2, gamma = 2 * 2 sigmoid(0) = 2;
    S_1 = (1 - k^2 b) alpha s + k w v, o = gamma q S_1. With k = 1, v = 4,
    q = 1/2, s = 6: S_1 = 0 + 2 = 2, o = 2."""
    o, S = oracle.muir_recurrent(_one(0.5), _one(1.0), _one(4.0), _one(0.0), _one(0.0), _one(0.0), [0.0],
                                 _one(0.0), np.full((1, 1), 2.0), S0=np.full((1, 1, 1, 1), 6.0))
    assert S.item() == 2.0 and o.item() == 2.0


@pytest.mark.parametrize("seed", range(3))
def test_decode_matches_recurrence(seed):
    d = muir_inputs(2, 2, 5, 4, 3, seed=seed, dtype="f32", s0_std=0.5)
    o_ref, S_ref = oracle.muir_recurrent(d["q"], d["k"], d["v"], d["z_f"], d["z_b"], d["z_w"], d["a_log"],
                                         d["z_q"], d["gamma_stat"], S0=d["S0"])
    S = d["S0"]
    for t in range(5):
        sl = lambda x: x[:, :, t]
        o, S = oracle.muir_decode(S, *(sl(d[n]) for n in ("q", "k", "v", "z_f", "z_b", "z_w")), d["a_log"],
                                  sl(d["z_q"]), d["gamma_stat"])
        assert _rel(o, o_ref[:, :, t]) < 1e-14
    assert _rel(S, S_ref) < 1e-14
