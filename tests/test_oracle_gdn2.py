"""Pins of the GDN-2 oracle against what the pages and the mathematics fix (CPU only).

Page: "Muir: Linear Attention with Sensitivity-Allocated Gating and
Matched-Filter Readout" (§2.1 eq.(1), §2.2) and "Exponential gates and matrix
memory: xLSTM and RWKV-7" (§13.2, §13.3).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import gdn2 as G
from synth import gdn2_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, B=2, H=2, T=9, dk=5, dv=4, alpha_mu=1.0, alpha_sigma=1.0, s0=0.5):
    d = gdn2_inputs(B, H, T, dk, dv, alpha_mu=alpha_mu, alpha_sigma=alpha_sigma,
                    seed=seed, dtype="f32", s0_std=s0)
    return d


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# --------------------------------------------------------------------------- worked example

def _load_two_steps():
    with open(os.path.join(GOLD, "gdn2_two_steps.json")) as f:
        g = json.load(f)
    fr = lambda m: [[Fraction(x) for x in r] for r in m]
    return g, fr


def test_hand_worked_two_steps():
    g, fr = _load_two_steps()
    arr = lambda key: np.array([[float(x) for x in r] for r in fr(g[key])])[None, None]
    o, S = oracle.gdn2_recurrent(arr("q"), arr("k"), arr("v"), arr("alpha"), arr("b"), arr("w"),
                                 S0=np.array([[float(x) for x in r] for r in fr(g["S0"])])[None, None])
    np.testing.assert_allclose(o[0, 0], np.array([[float(x) for x in r] for r in fr(g["o"])]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(S[0, 0], np.array([[float(x) for x in r] for r in fr(g["S_T"])]), rtol=0, atol=1e-15)


def test_bruteforce_exact_reproduces_hand_example():
    g, fr = _load_two_steps()
    o, S = oracle.bruteforce_exact(fr(g["q"]), fr(g["k"]), fr(g["v"]), fr(g["alpha"]), fr(g["b"]),
                                   fr(g["w"]), fr(g["S0"]))
    assert o == fr(g["o"])
    assert S == fr(g["S_T"])


# --------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("T,dk,dv", [(1, 2, 3), (3, 3, 2), (6, 4, 4), (8, 2, 2)])
def test_bruteforce_exact_dyadic(seed, T, dk, dv):
    """Exact rational transition products on dyadic inputs vs the float64 recurrence."""
    rng = np.random.default_rng(1000 + seed)
    dy = lambda shape, lo, hi, den=16: rng.integers(lo, hi, size=shape) / den
    q, k = dy((T, dk), -16, 17), dy((T, dk), -16, 17)
    v, S0 = dy((T, dv), -32, 33), dy((dk, dv), -16, 17)
    alpha, b, w = dy((T, dk), 1, 17), dy((T, dk), 0, 33), dy((T, dv), 0, 17)
    o_ex, S_ex = oracle.bruteforce_exact(q, k, v, alpha, b, w, S0)
    o, S = oracle.gdn2_recurrent(q[None, None], k[None, None], v[None, None], alpha[None, None],
                                 b[None, None], w[None, None], S0=S0[None, None])
    o_ex = np.array([[float(x) for x in r] for r in o_ex])
    S_ex = np.array([[float(x) for x in r] for r in S_ex])
    scale = max(1.0, np.abs(o_ex).max(), np.abs(S_ex).max())
    assert np.abs(o[0, 0] - o_ex).max() <= 1e-14 * scale
    assert np.abs(S[0, 0] - S_ex).max() <= 1e-14 * scale


# --------------------------------------------------------------------------- alternative forms

@pytest.mark.parametrize("seed", range(3))
def test_materialized_transition_matches_rank_one_step(seed):
    """Rank-one step vs the explicit dk x dk transition loop (the pages pin 5.3e-15)."""
    d = _rand(seed)
    args = [d[x] for x in ("q", "k", "v", "alpha", "b", "w")]
    o1, S1 = oracle.gdn2_recurrent(*args, S0=d["S0"])
    o2, S2 = oracle.gdn2_materialized(*args, S0=d["S0"])
    assert _rel(o1, o2) < 1e-14 and _rel(S1, S2) < 1e-14


@pytest.mark.parametrize("seed", range(3))
def test_effective_write_form(seed):
    """§2.2: S_t = Diag(alpha_t) S_{t-1} + k_t^T v_tilde_t with v_tilde_t = v_hat_t - k_hat_t Diag(alpha_t) S_{t-1}."""
    d = _rand(seed)
    args = [d[x] for x in ("q", "k", "v", "alpha", "b", "w")]
    o1, S1 = oracle.gdn2_recurrent(*args, S0=d["S0"])
    o2, S2 = oracle.gdn2_effective_write(*args, S0=d["S0"])
    assert _rel(o1, o2) < 1e-14 and _rel(S1, S2) < 1e-14


def test_t1_closed_form():
    """From S0 = 0 one token gives S_1 = k^T (w*v) and o_1 = (q.k)(w*v)."""
    d = _rand(7, T=1, s0=None)
    o, S = oracle.gdn2_recurrent(*[d[x] for x in ("q", "k", "v", "alpha", "b", "w")])
    vh = d["w"][:, :, 0] * d["v"][:, :, 0]
    qk = np.sum(d["q"][:, :, 0] * d["k"][:, :, 0], axis=-1)
    np.testing.assert_allclose(S, d["k"][:, :, 0, :, None] * vh[:, :, None, :], rtol=0, atol=1e-16)
    np.testing.assert_allclose(o[:, :, 0], qk[..., None] * vh, rtol=0, atol=1e-15)


def test_erase_contracts_along_k_with_eigenvalue():
    """§2.1: I - k^T (b*k) maps the rank-one state k^T x to (1 - <k, b*k>) k^T x."""
    rng = np.random.default_rng(3)
    dk, dv = 6, 3
    k = rng.standard_normal(dk); k /= np.linalg.norm(k)
    b = rng.uniform(0.1, 1.9, dk)
    x = rng.standard_normal(dv)
    S0 = np.outer(k, x)
    one = lambda a: a[None, None, None]
    _, S = oracle.gdn2_recurrent(one(np.zeros(dk)), one(k), one(np.zeros(dv)), one(np.ones(dk)),
                                 one(b), one(np.zeros(dv)), S0=S0[None, None])
    lam = 1.0 - np.dot(k, b * k)
    np.testing.assert_allclose(S[0, 0], lam * S0, rtol=0, atol=1e-15)


def test_split_sequence_state_passing():
    d = _rand(11, T=12)
    a = [d[x] for x in ("q", "k", "v", "alpha", "b", "w")]
    o, S = oracle.gdn2_recurrent(*a, S0=d["S0"])
    oA, SA = oracle.gdn2_recurrent(*[x[:, :, :5] for x in a], S0=d["S0"])
    oB, SB = oracle.gdn2_recurrent(*[x[:, :, 5:] for x in a], S0=SA)
    np.testing.assert_allclose(np.concatenate([oA, oB], axis=2), o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(SB, S, rtol=0, atol=1e-14)


def test_decode_steps_equal_recurrent():
    d = _rand(12, T=7)
    a = [d[x] for x in ("q", "k", "v", "alpha", "b", "w")]
    o, S = oracle.gdn2_recurrent(*a, S0=d["S0"])
    St = d["S0"]
    for t in range(7):
        ot, St = oracle.gdn2_decode(St, *[x[:, :, t] for x in a])
        np.testing.assert_allclose(ot, o[:, :, t], rtol=0, atol=1e-14)
    np.testing.assert_allclose(St, S, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- reductions

@pytest.mark.parametrize("seed", range(3))
def test_reduces_to_plain_delta_rule(seed):
    """alpha = 1 and b = w = beta_t 1: the delta rule S <- S - beta k^T (k S - v)."""
    d = _rand(seed)
    beta = np.random.default_rng(seed).uniform(0.05, 1.5, d["q"].shape[:3])
    bb = np.broadcast_to(beta[..., None], d["q"].shape)
    bw = np.broadcast_to(beta[..., None], d["v"].shape)
    o1, S1 = oracle.gdn2_recurrent(d["q"], d["k"], d["v"], np.ones_like(d["q"]), bb, bw, S0=d["S0"])
    o2, S2 = oracle.delta_rule_textbook(d["q"], d["k"], d["v"], beta, S0=d["S0"])
    assert _rel(o1, o2) < 1e-14 and _rel(S1, S2) < 1e-14


def test_delta_rule_is_online_gradient_step():
    """Same reduction checked against autograd's gradient of 0.5*||k S - v||^2 (float64, CPU)."""
    rng = np.random.default_rng(5)
    dk, dv, T = 5, 3, 6
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.1, 1.0, T)
    S0 = rng.standard_normal((dk, dv))
    S = torch.tensor(S0, dtype=torch.float64)
    for t in range(T):
        St = S.clone().requires_grad_(True)
        loss = 0.5 * torch.sum((torch.tensor(k[t]) @ St - torch.tensor(v[t])) ** 2)
        (g,) = torch.autograd.grad(loss, St)
        S = (St - beta[t] * g).detach()
    one = lambda x: x[None, None]
    _, S_or = oracle.gdn2_recurrent(one(np.zeros((T, dk))), one(k), one(v), one(np.ones((T, dk))),
                                    one(np.repeat(beta[:, None], dk, 1)), one(np.repeat(beta[:, None], dv, 1)),
                                    S0=one(S0))
    np.testing.assert_allclose(S_or[0, 0], S.numpy(), rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_reduces_to_gated_deltanet(seed):
    """alpha = gamma_t 1, b = w = beta_t 1 (the pages pin this reduction at 8.9e-16)."""
    d = _rand(seed)
    rng = np.random.default_rng(50 + seed)
    gamma = rng.uniform(0.3, 1.0, d["q"].shape[:3])
    beta = rng.uniform(0.05, 1.5, d["q"].shape[:3])
    ex = lambda x, like: np.broadcast_to(x[..., None], like.shape)
    o1, S1 = oracle.gdn2_recurrent(d["q"], d["k"], d["v"], ex(gamma, d["q"]), ex(beta, d["q"]),
                                   ex(beta, d["v"]), S0=d["S0"])
    o2, S2 = oracle.gated_deltanet(d["q"], d["k"], d["v"], gamma, beta, S0=d["S0"])
    assert _rel(o1, o2) < 1e-14 and _rel(S1, S2) < 1e-14


@pytest.mark.parametrize("seed", range(3))
def test_reduces_to_gla_when_no_erase(seed):
    d = _rand(seed, T=10)
    o1, S1 = oracle.gdn2_recurrent(d["q"], d["k"], d["v"], d["alpha"], np.zeros_like(d["b"]), d["w"], S0=d["S0"])
    o2, S2 = oracle.gla_closed_form(d["q"], d["k"], d["v"], d["alpha"], d["w"], S0=d["S0"])
    assert _rel(o1, o2) < 1e-13 and _rel(S1, S2) < 1e-13


def test_reduces_to_linear_attention():
    d = _rand(4, T=10)
    one = np.ones_like(d["q"])
    o1, S1 = oracle.gdn2_recurrent(d["q"], d["k"], d["v"], one, 0 * one, np.ones_like(d["v"]), S0=d["S0"])
    o2, S2 = oracle.linear_attention_closed_form(d["q"], d["k"], d["v"], S0=d["S0"])
    assert _rel(o1, o2) < 1e-13 and _rel(S1, S2) < 1e-13


# --------------------------------------------------------------------------- mutations are caught

def _mutants():
    def erase_before_decay(S, q, k, v, alpha, b, w):
        read = np.einsum("...i,...ij->...j", b * k, S)
        S2 = alpha[..., :, None] * (S - k[..., :, None] * read[..., None, :]) + k[..., :, None] * (w * v)[..., None, :]
        return np.einsum("...i,...ij->...j", q, S2), S2

    def transposed_rank_one(S, q, k, v, alpha, b, w):
        Sh = alpha[..., :, None] * S
        read = np.einsum("...i,...ij->...j", k, Sh)
        S2 = Sh - (b * k)[..., :, None] * read[..., None, :] + k[..., :, None] * (w * v)[..., None, :]
        return np.einsum("...i,...ij->...j", q, S2), S2

    def readout_before_write(S, q, k, v, alpha, b, w):
        Sh = alpha[..., :, None] * S
        o = np.einsum("...i,...ij->...j", q, S)
        read = np.einsum("...i,...ij->...j", b * k, Sh)
        return o, Sh - k[..., :, None] * read[..., None, :] + k[..., :, None] * (w * v)[..., None, :]

    def sign_flip_erase(S, q, k, v, alpha, b, w):
        Sh = alpha[..., :, None] * S
        read = np.einsum("...i,...ij->...j", b * k, Sh)
        S2 = Sh + k[..., :, None] * read[..., None, :] + k[..., :, None] * (w * v)[..., None, :]
        return np.einsum("...i,...ij->...j", q, S2), S2

    def dropped_write_gate(S, q, k, v, alpha, b, w):
        Sh = alpha[..., :, None] * S
        read = np.einsum("...i,...ij->...j", b * k, Sh)
        S2 = Sh - k[..., :, None] * read[..., None, :] + k[..., :, None] * v[..., None, :]
        return np.einsum("...i,...ij->...j", q, S2), S2

    def decay_after_write(S, q, k, v, alpha, b, w):
        read = np.einsum("...i,...ij->...j", b * k, S)
        S2 = alpha[..., :, None] * (S - k[..., :, None] * read[..., None, :] + k[..., :, None] * (w * v)[..., None, :])
        return np.einsum("...i,...ij->...j", q, S2), S2

    def erase_reads_undecayed(S, q, k, v, alpha, b, w):
        Sh = alpha[..., :, None] * S
        read = np.einsum("...i,...ij->...j", b * k, S)
        S2 = Sh - k[..., :, None] * read[..., None, :] + k[..., :, None] * (w * v)[..., None, :]
        return np.einsum("...i,...ij->...j", q, S2), S2

    def erase_gate_on_both_sides(S, q, k, v, alpha, b, w):
        Sh = alpha[..., :, None] * S
        read = np.einsum("...i,...ij->...j", b * k, Sh)
        S2 = Sh - (b * k)[..., :, None] * read[..., None, :] + k[..., :, None] * (w * v)[..., None, :]
        return np.einsum("...i,...ij->...j", q, S2), S2

    return [erase_before_decay, transposed_rank_one, readout_before_write, sign_flip_erase,
            dropped_write_gate, decay_after_write, erase_reads_undecayed, erase_gate_on_both_sides]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_pins_reject_planted_mistakes(monkeypatch, mutant):
    """Each planted oracle mistake must fail a pin: the hand-worked example,
    or the exact rational brute force on random dyadic inputs (the hand
    example's erase gate cannot tell (b*k)^T (b*k) from k^T (b*k))."""
    monkeypatch.setattr(G, "gdn2_step", mutant)

    def pins():
        test_hand_worked_two_steps()
        for seed in range(3):
            test_bruteforce_exact_dyadic(seed, 5, 3, 2)

    with pytest.raises(AssertionError):
        pins()


def test_pins_pass_the_unmutated_step():
    """Control for the planted-mistake test: the same pins pass as written."""
    test_hand_worked_two_steps()
    for seed in range(3):
        test_bruteforce_exact_dyadic(seed, 5, 3, 2)


# --------------------------------------------------------------------------- chunkwise form

@pytest.mark.parametrize("chunk,T", [(4, 16), (8, 21), (16, 16), (5, 1)])
def test_chunkwise_form_equals_recurrence(chunk, T):
    """The Muir page's eq.(10) (T [U|Y] = [V_hat|K_hat_pi], O = (Q_pi - M Y) S0 + M U,
    S_C = (Diag(pi_C) - K_tilde^T Y) S0 + K_tilde^T U) reproduces eq.(1) step by
    step, including a ragged last chunk."""
    d = _rand(40 + chunk, T=T, dk=6, dv=5, alpha_mu=1.5)
    o1, S1 = oracle.gdn2_recurrent(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], S0=d["S0"])
    o2, S2 = G.gdn2_chunkwise(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], S0=d["S0"], chunk=chunk)
    assert _rel(o2, o1) < 1e-13 and _rel(S2, S1) < 1e-13


def test_chunk_system_is_identity_without_erase():
    """b = 0: no erase term, the chunk matrix is I and its condition number 1."""
    d = _rand(50, T=12, dk=4, dv=3)
    mats = G.gdn2_chunk_system(d["k"], d["alpha"], np.zeros_like(d["b"]), 8)
    for m in mats:
        assert np.array_equal(m, np.broadcast_to(np.eye(m.shape[-1]), m.shape))
    kap = G.chunk_condition_numbers(d["k"], d["alpha"], np.zeros_like(d["b"]), 8)
    assert np.allclose(kap, 1.0)


def test_chunk_system_two_tokens_closed_form():
    """Two tokens: T = [[1, 0], [<b_2*k_2, alpha_2*k_1>, 1]] (pi_{2,1} = alpha_2)."""
    k = np.array([[[[0.6, 0.8], [1.0, 0.0]]]])
    alpha = np.array([[[[0.5, 0.25], [0.5, 0.25]]]])
    b = np.array([[[[1.0, 2.0], [1.5, 0.5]]]])
    (m,) = G.gdn2_chunk_system(k, alpha, b, 2)
    l21 = 1.5 * 1.0 * 0.5 * 0.6 + 0.5 * 0.0 * 0.25 * 0.8
    assert np.allclose(m[0, 0], [[1.0, 0.0], [l21, 1.0]], rtol=0, atol=1e-15)


def test_chunkwise_solve_catches_a_planted_transpose():
    """Solving with T^T instead of T (a plausible slip) breaks the agreement."""
    d = _rand(60, T=16, dk=5, dv=4, alpha_mu=1.5)
    orig = G.gdn2_chunk_system
    try:
        G.gdn2_chunk_system = lambda *a: [np.swapaxes(m, -1, -2) for m in orig(*a)]
        o2, _ = G.gdn2_chunkwise(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], S0=d["S0"], chunk=8)
    finally:
        G.gdn2_chunk_system = orig
    o1, _ = oracle.gdn2_recurrent(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], S0=d["S0"])
    assert _rel(o2, o1) > 1e-3
