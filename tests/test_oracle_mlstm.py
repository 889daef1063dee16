"""Pins of the mLSTM oracle (CPU only).

Page: "Exponential gates and matrix memory: xLSTM and RWKV-7", §13.4, Prop. 13.3
and the solution to Exercise 13.6.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import mlstm_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _pin(name):
    with open(os.path.join(GOLD, "pages_pins.json")) as f:
        return next(p for p in json.load(f)["pins"] if p["name"] == name)


def test_hand_worked_two_steps():
    with open(os.path.join(GOLD, "mlstm_two_steps.json")) as f:
        g = json.load(f)
    m = lambda key: np.array([[float(Fraction(x)) for x in r] for r in g[key]])
    i_t = np.array([math.log(float(x)) for x in g["i_tilde_log"]])
    f_t = np.array([float(x) for x in g["f_tilde"]])
    h, C, n, mT = oracle.mlstm_stabilized(m("q")[None, None], m("k")[None, None], m("v")[None, None],
                                          i_t[None, None], f_t[None, None])
    np.testing.assert_allclose(h[0, 0], m("h"), rtol=1e-15, atol=0)
    np.testing.assert_allclose(C[0, 0], m("C_T"), rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(n[0, 0], [float(Fraction(x)) for x in g["n_T"]], rtol=1e-15, atol=1e-15)
    assert abs(mT[0, 0] - math.log(float(g["m_T_log"]))) < 1e-15


@pytest.mark.parametrize("i_tilde", [0.0, 100.0, 800.0])
def test_single_pair_recovery(i_tilde):
    """One write of v on a unit key, read at q = k, returns v for any input log-gate."""
    pin = _pin("mlstm_single_pair_recovery")
    v = np.array(pin["v"])
    rng = np.random.default_rng(1)
    k = rng.standard_normal(5); k /= np.linalg.norm(k)
    one = lambda x: np.asarray(x)[None, None, None]
    h, _, _, _ = oracle.mlstm_stabilized(one(k), one(k), one(v), one(i_tilde), one(2.0))
    assert np.abs(h[0, 0, 0] - v).max() <= 1e-15
    hn, _, _ = oracle.mlstm_naive(one(k), one(k), one(v), one(i_tilde), one(2.0))
    if i_tilde >= pin["i_tilde"]:
        assert not np.all(np.isfinite(hn))       # exp(800) overflows float64
    else:
        assert np.abs(hn[0, 0, 0] - v).max() <= 1e-14


@pytest.mark.parametrize("seed", range(3))
def test_stabilized_equals_naive_in_safe_regime(seed):
    d = mlstm_inputs(2, 2, 40, 6, 5, seed=seed, dtype="f32")
    h1, C, n, m = oracle.mlstm_stabilized(d["q"], d["k"], d["v"], d["i_tilde"], d["f_tilde"])
    h2, C2, n2 = oracle.mlstm_naive(d["q"], d["k"], d["v"], d["i_tilde"], d["f_tilde"])
    assert np.linalg.norm(h1 - h2) / np.linalg.norm(h2) < 1e-13
    # the scaled state is the raw state times exp(-m_T)
    np.testing.assert_allclose(C * np.exp(m)[..., None, None], C2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(n * np.exp(m)[..., None], n2, rtol=1e-12, atol=1e-12)


def test_overflow_cliff():
    pin = _pin("mlstm_overflow_cliff")
    rng = np.random.default_rng(2)
    T, dk, dv = 12, 4, 3
    q = rng.standard_normal((T, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    f_t = np.full(T, 3.0)
    one = lambda x: x[None, None]
    for gate, naive_ok in ((pin["naive_finite_at"], True), (pin["naive_nan_at"], False)):
        i_t = np.zeros(T); i_t[5] = gate
        hs, C, n, m = oracle.mlstm_stabilized(one(q), one(k), one(v), one(i_t), one(f_t))
        hn, Cn, _ = oracle.mlstm_naive(one(q), one(k), one(v), one(i_t), one(f_t))
        assert np.all(np.isfinite(hs)) and np.abs(C).max() <= T
        if naive_ok:
            assert np.all(np.isfinite(hn)) and np.abs(Cn).max() > 1e300
            assert np.linalg.norm(hs - hn) / np.linalg.norm(hs) < 1e-14
        else:
            assert np.isnan(hn).any()
    assert math.log(np.finfo(np.float64).max) == pytest.approx(pin["float64_exp_limit"], abs=1e-2)


def test_scaled_gates_in_unit_interval():
    d = mlstm_inputs(1, 3, 50, 4, 4, seed=3, dtype="f32")
    logf = oracle.log_sigmoid(d["f_tilde"])
    m = np.empty_like(d["i_tilde"])
    prev = np.full(m.shape[:2], -np.inf)
    for t in range(m.shape[-1]):     # the running max as the page defines it
        prev = m[..., t] = np.maximum(logf[..., t] + prev, d["i_tilde"][..., t])
    fp = np.exp(logf[..., 1:] + m[..., :-1] - m[..., 1:])
    ip = np.exp(d["i_tilde"] - m)
    assert np.all((fp > 0) & (fp <= 1)) and np.all((ip > 0) & (ip <= 1))


@pytest.mark.parametrize("seed", range(3))
def test_closed_form_stabilizer_matches_recurrence(seed):
    d = mlstm_inputs(2, 2, 30, 3, 3, seed=seed, dtype="f32")
    mc = oracle.stabilizer_closed_form(d["i_tilde"], d["f_tilde"])
    logf = oracle.log_sigmoid(d["f_tilde"])
    m = np.full(d["i_tilde"].shape[:2], -np.inf)
    for t in range(30):
        m = np.maximum(logf[..., t] + m, d["i_tilde"][..., t])
        np.testing.assert_allclose(mc[..., t], m, rtol=0, atol=1e-13)
    m0 = np.array([[1.5, -2.0], [0.0, 7.0]])
    mc0 = oracle.stabilizer_closed_form(d["i_tilde"], d["f_tilde"], m0=m0)
    m = m0.copy()
    for t in range(30):
        m = np.maximum(logf[..., t] + m, d["i_tilde"][..., t])
    np.testing.assert_allclose(mc0[..., -1], m, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_readout_invariant_to_stabilizer_choice(seed):
    """Exercise 13.6: the stabiliser is a change of variables, so any stabiliser
    sequence that keeps the arithmetic in range gives the same readout."""
    d = mlstm_inputs(1, 2, 25, 4, 3, seed=seed, dtype="f32")
    h_ref, _, _, _ = oracle.mlstm_stabilized(d["q"], d["k"], d["v"], d["i_tilde"], d["f_tilde"])
    m = oracle.stabilizer_closed_form(d["i_tilde"], d["f_tilde"])
    rng = np.random.default_rng(seed)
    for m_alt in (m + 3.0, m - 2.5, m + rng.uniform(-1, 4, m.shape)):
        h = oracle.mlstm_with_stabilizer(d["q"], d["k"], d["v"], d["i_tilde"], d["f_tilde"], m_alt)
        assert np.linalg.norm(h - h_ref) / np.linalg.norm(h_ref) < 1e-13


@pytest.mark.parametrize("seed", range(2))
def test_returned_stabilizer_matches_closed_form(seed):
    """The stabiliser the recurrence carries (and returns) is the running max
    of §13.4, here against its independent prefix-max closed form (the readout
    alone does not fix it: any stabiliser gives the same h while the floor is
    inactive)."""
    d = mlstm_inputs(2, 2, 30, 4, 3, seed=seed, dtype="f32")
    _, _, _, m = oracle.mlstm_stabilized(d["q"], d["k"], d["v"], d["i_tilde"], d["f_tilde"])
    mc = oracle.stabilizer_closed_form(d["i_tilde"], d["f_tilde"])
    np.testing.assert_allclose(m, mc[..., -1], rtol=0, atol=1e-12)


def test_nonempty_initial_state_continues_sequence():
    d = mlstm_inputs(2, 2, 20, 4, 3, seed=9, dtype="f32")
    a = [d[x] for x in ("q", "k", "v", "i_tilde", "f_tilde")]
    h, C, n, m = oracle.mlstm_stabilized(*a)
    h1, C1, n1, m1 = oracle.mlstm_stabilized(*[x[:, :, :8] for x in a])
    h2, C2, n2, m2 = oracle.mlstm_stabilized(*[x[:, :, 8:] for x in a], C0=C1, n0=n1, m0=m1)
    np.testing.assert_allclose(np.concatenate([h1, h2], axis=2), h, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(C2, C, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(m2, m, rtol=0, atol=1e-13)


# --------------------------------------------------------------------------- mutations are caught

def _stabilized_variant(mistake):
    """The stabilised recurrence restated with one planted mistake (test code:
    each variant must make at least one pin above fail)."""
    def run(q, k, v, i_tilde, f_tilde, C0=None, n0=None, m0=None):
        q, k, v, i_tilde, f_tilde = (np.asarray(x, dtype=np.float64) for x in (q, k, v, i_tilde, f_tilde))
        B, H, T, dk = q.shape
        C = np.zeros((B, H, dk, v.shape[-1])) if C0 is None else np.array(C0, dtype=np.float64)
        n = np.zeros((B, H, dk)) if n0 is None else np.array(n0, dtype=np.float64)
        m = np.full((B, H), -np.inf) if m0 is None else np.array(m0, dtype=np.float64)
        logf = oracle.log_sigmoid(f_tilde)
        h = np.zeros(v.shape)
        for t in range(T):
            lf = 0.0 if mistake == "stabiliser_without_forget" else logf[:, :, t]
            m_new = np.maximum(lf + m, i_tilde[:, :, t])
            with np.errstate(invalid="ignore", over="ignore"):
                fp = np.exp(logf[:, :, t] + m - m_new)
            fp = np.where(np.isneginf(m), 0.0, fp)
            ip = np.exp(i_tilde[:, :, t] - m_new)
            if mistake == "forget_gate_on_write":
                ip = ip * np.exp(logf[:, :, t])
            C_prev = C
            C = fp[..., None, None] * C + ip[..., None, None] * k[:, :, t, :, None] * v[:, :, t, None, :]
            n = fp[..., None] * n + (1.0 if mistake == "unscaled_normaliser_write" else ip[..., None]) * k[:, :, t]
            m = m_new
            Cr = C_prev if mistake == "readout_before_write" else C
            num = np.einsum("bhi,bhij->bhj", q[:, :, t], Cr)
            qn = np.sum(q[:, :, t] * n, axis=-1)
            floor = 1.0 if mistake == "unscaled_floor" else np.exp(-m)
            den = np.maximum(qn if mistake == "no_abs_in_normaliser" else np.abs(qn), floor)
            h[:, :, t] = num / den[..., None]
        return h, C, n, m
    return run


MISTAKES = ["stabiliser_without_forget", "forget_gate_on_write", "unscaled_normaliser_write",
            "readout_before_write", "unscaled_floor", "no_abs_in_normaliser"]


def _run_pins():
    test_hand_worked_two_steps()
    for it in (0.0, 100.0, 800.0):
        test_single_pair_recovery(it)
    for seed in range(3):
        test_stabilized_equals_naive_in_safe_regime(seed)
    test_overflow_cliff()
    for seed in range(2):
        test_returned_stabilizer_matches_closed_form(seed)
    test_nonempty_initial_state_continues_sequence()


def test_restated_recurrence_passes_the_pins(monkeypatch):
    """Control: the restatement without a mistake passes every pin."""
    monkeypatch.setattr(oracle, "mlstm_stabilized", _stabilized_variant(None))
    _run_pins()


@pytest.mark.parametrize("mistake", MISTAKES)
def test_pins_reject_planted_mistakes(monkeypatch, mistake):
    monkeypatch.setattr(oracle, "mlstm_stabilized", _stabilized_variant(mistake))
    with pytest.raises(AssertionError):
        _run_pins()
