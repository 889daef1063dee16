"""Pins of the RWKV-7 generalized delta-rule oracle (CPU only).

Page: "Exponential gates and matrix memory: xLSTM and RWKV-7", §13.2-§13.3 and
the solution to Exercise 13.5.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import rwkv7 as R

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _pin(name):
    with open(os.path.join(GOLD, "pages_pins.json")) as f:
        return next(p for p in json.load(f)["pins"] if p["name"] == name)


def _rand(seed, B=2, H=2, T=9, dk=5, dv=4):
    rng = np.random.default_rng(seed)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    return dict(q=rng.standard_normal((B, H, T, dk)), w=rng.uniform(0.3, 1.0, (B, H, T, dk)),
                a=unit(rng.standard_normal((B, H, T, dk))), c=rng.uniform(0, 1.5, (B, H, T)),
                kw=rng.standard_normal((B, H, T, dk)) * 0.5, u=rng.standard_normal((B, H, T, dv)),
                S0=rng.standard_normal((B, H, dk, dv)) * 0.3)


def _rel(x, y):
    return np.linalg.norm(x - y) / np.linalg.norm(y)


@pytest.mark.parametrize("seed", range(3))
def test_rank_one_form_matches_materialized_transitions(seed):
    """Page: rank-one scan vs materialised-transition loop, 5.3e-15."""
    d = _rand(seed)
    args = [d[n] for n in ("q", "w", "a", "c", "kw", "u")]
    o1, S1 = R.rwkv7_recurrent(*args, S0=d["S0"])
    o2, S2 = R.rwkv7_materialized(*args, S0=d["S0"])
    assert _rel(o1, o2) < 1e-13 and _rel(S1, S2) < 1e-13


@pytest.mark.parametrize("seed", range(3))
def test_reduces_to_gated_deltanet(seed):
    """Solution to Exercise 13.5: w = gamma 1, a = k/|k|, c = gamma beta |k|^2 and
    the write u b^T = beta v k^T give Gated DeltaNet (page: 8.9e-16)."""
    rng = np.random.default_rng(50 + seed)
    B, H, T, dk, dv = 1, 2, 8, 4, 3
    q, k = rng.standard_normal((B, H, T, dk)), rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    gamma, beta = rng.uniform(0.5, 1, (B, H, T)), rng.uniform(0, 1, (B, H, T))
    nk = np.linalg.norm(k, axis=-1)
    S0 = rng.standard_normal((B, H, dk, dv))
    o1, S1 = R.rwkv7_recurrent(q, np.broadcast_to(gamma[..., None], k.shape), k / nk[..., None],
                               gamma * beta * nk ** 2, k, beta[..., None] * v, S0=S0)
    o2, S2 = oracle.gated_deltanet(q, k, v, gamma, beta, S0=S0)
    assert np.abs(o1 - o2).max() < 1e-13 and np.abs(S1 - S2).max() < 1e-13


@pytest.mark.parametrize("c", [0.1, 0.37])
def test_decoupled_eviction(c):
    """§13.3: store (k_A, v_A) on a unit key, then T writes on keys orthogonal to
    k_A. Removal aimed at k_A decays the retrieval k_A S_T as (1 - c)^T |v_A|;
    removal locked to the write key leaves it at |v_A|. The page's numbers at
    c = 0.1, T = 30: 0.028576 against a flat 0.674096."""
    pin = _pin("decoupled_eviction")
    T, dk, dv = pin["T"], 8, 5
    rng = np.random.default_rng(3)
    kA = np.zeros(dk)
    kA[0] = 1.0
    vA = rng.standard_normal(dv)
    vA *= pin["locked_norm"] / np.linalg.norm(vA)         # |v_A| as on the page
    keys = rng.standard_normal((T, dk))
    keys[:, 0] = 0.0                                        # orthogonal to k_A
    keys /= np.linalg.norm(keys, axis=-1, keepdims=True)
    S0 = np.outer(kA, vA)[None, None]                       # the stored association
    sh = lambda x: x[None, None]
    ones = np.ones((T, dk))
    vals = rng.standard_normal((T, dv))
    cc = np.full((T,), c)
    _, S_aim = R.rwkv7_recurrent(sh(np.zeros((T, dk))), sh(ones), sh(np.tile(kA, (T, 1))), sh(cc),
                                 sh(keys), sh(vals), S0=S0)
    _, S_lock = R.rwkv7_recurrent(sh(np.zeros((T, dk))), sh(ones), sh(keys), sh(cc), sh(keys), sh(vals), S0=S0)
    aimed = np.linalg.norm(kA @ S_aim[0, 0])
    locked = np.linalg.norm(kA @ S_lock[0, 0])
    assert abs(aimed - (1 - c) ** T * pin["locked_norm"]) < 1e-15
    assert abs(locked - pin["locked_norm"]) < 1e-15
    if c == pin["c"]:
        assert round(aimed, 6) == pin["aimed_norm"]


def test_decode_matches_recurrence():
    d = _rand(7, T=5)
    o_ref, S_ref = R.rwkv7_recurrent(*(d[n] for n in ("q", "w", "a", "c", "kw", "u")), S0=d["S0"])
    S = d["S0"]
    for t in range(5):
        o, S = R.rwkv7_decode(S, *(d[n][:, :, t] for n in ("q", "w", "a", "c", "kw", "u")))
        assert _rel(o, o_ref[:, :, t]) < 1e-14
    assert _rel(S, S_ref) < 1e-14


def test_planted_mistake_removal_reading_the_decayed_state():
    """Reading the removal on Diag(w) S instead of S (GDN-2's order) changes the
    result: the pins above would catch such a slip."""
    d = _rand(8)
    args = [d[n] for n in ("q", "w", "a", "c", "kw", "u")]
    o1, _ = R.rwkv7_recurrent(*args, S0=d["S0"])
    orig = R.rwkv7_step

    def wrong(S, q, w, a, c, kw, u):
        return orig(w[..., :, None] * S, q, np.ones_like(w), a, c, kw, u)
    try:
        R.rwkv7_step = wrong
        o2, _ = R.rwkv7_recurrent(*args, S0=d["S0"])
    finally:
        R.rwkv7_step = orig
    assert _rel(o2, o1) > 1e-3
