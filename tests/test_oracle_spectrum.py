"""Pins of the transition's spectrum (CPU only).

Page: "Exponential gates and matrix memory: xLSTM and RWKV-7", §13.2, Prop. 13.1,
Exercises 13.1 and 13.4. The GDN-2 transition of "Muir: ...", §2.1 eq.(1),
A = (I - k^T (b*k)) Diag(alpha), is materialised by the oracle and checked here.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _unit(rng, d):
    x = rng.standard_normal(d)
    return x / np.linalg.norm(x)


@pytest.mark.parametrize("seed", range(5))
def test_scalar_diagonal_spectrum_of_generalized_transition(seed):
    rng = np.random.default_rng(seed)
    d = 8
    a = _unit(rng, d)
    w0, c = rng.uniform(0.2, 1.0), rng.uniform(0.0, 2.5)
    ev = np.linalg.eigvalsh(oracle.generalized_transition(np.full(d, w0), c, a))
    np.testing.assert_allclose(ev, oracle.scalar_diagonal_spectrum(w0, c, d), rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed", range(5))
def test_gdn2_transition_scalar_decay_spectrum(seed):
    """alpha = alpha0 1: eig(A) = {alpha0 (1 - <k, b*k>)} and alpha0 (d-1 times)."""
    rng = np.random.default_rng(10 + seed)
    d = 8
    k = _unit(rng, d)
    alpha0 = rng.uniform(0.2, 1.0)
    for b in (np.full(d, rng.uniform(0.0, 2.0)), rng.uniform(0.0, 2.0, d)):
        A = oracle.gdn2_transition(k, np.full(d, alpha0), b)
        ev = np.sort(np.linalg.eigvals(A).real)
        expect = np.sort(np.array([alpha0 * (1.0 - np.dot(k, b * k))] + [alpha0] * (d - 1)))
        np.testing.assert_allclose(ev, expect, rtol=0, atol=1e-14)
        if np.all(b == b[0]):   # A is symmetric when the erase gate is scalar
            np.testing.assert_allclose(np.linalg.eigvalsh(A), expect, rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed", range(5))
def test_gdn2_transition_channelwise_spectrum(seed):
    """Channel-wise alpha, b: A is similar to the symmetric Diag(alpha) - c^T c, c = sqrt(alpha*b)*k,
    so its eigenvalues are real, solve the secular equation and interlace the alphas."""
    rng = np.random.default_rng(20 + seed)
    d = 7
    k = _unit(rng, d)
    alpha = np.sort(rng.uniform(0.1, 1.0, d))
    b = rng.uniform(0.05, 1.95, d)
    A = oracle.gdn2_transition(k, alpha, b)
    Msym, c = oracle.symmetrized_transition(k, alpha, b)
    ev_sym = np.linalg.eigvalsh(Msym)
    ev = np.linalg.eigvals(A)
    assert np.abs(ev.imag).max() < 1e-12
    np.testing.assert_allclose(np.sort(ev.real), ev_sym, rtol=0, atol=1e-13)
    cn = np.dot(c, c)
    for lam in ev_sym:
        if np.min(np.abs(alpha - lam)) > 1e-6:
            assert abs(oracle.secular_residual(lam, alpha, cn, c / np.sqrt(cn))) < 1e-9
    assert ev_sym.min() >= alpha.min() - cn - 1e-12 and ev_sym.max() <= alpha.max() + 1e-12
    # interlacing: one eigenvalue in each gap between consecutive diagonal entries
    for i in range(d - 1):
        assert alpha[i] - 1e-12 <= ev_sym[i + 1] <= alpha[i + 1] + 1e-12


def test_exercise_13_1_spectral_radius():
    with open(os.path.join(GOLD, "pages_pins.json")) as f:
        pin = next(p for p in json.load(f)["pins"] if p["name"] == "exercise_13_1_spectral_radius")
    rng = np.random.default_rng(0)
    d = 6
    a = _unit(rng, d)
    for c, rho in zip(pin["c"], pin["rho"]):
        # through the GDN-2 oracle: alpha = 1, unit k = a, erase gate b = c 1
        A = oracle.gdn2_transition(a, np.ones(d), np.full(d, c))
        assert abs(np.max(np.abs(np.linalg.eigvals(A))) - rho) < 1e-12
