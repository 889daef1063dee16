"""Pins of the gradient oracle (CPU only): central finite differences of the
float64 forward recurrence, and closed forms where the recurrence reduces to
linear attention ("Muir: ...", §2.1 eq.(1); §4.2 "Custom Backward Pass")."""
import numpy as np
import pytest

import oracle
from oracle.gdn2_grad import gdn2_grad
from synth import gdn2_inputs

NAMES = ("q", "k", "v", "alpha", "b", "w")


def _loss(d, dO, dS, **over):
    x = {n: over.get(n, d[n]) for n in NAMES}
    S0 = over.get("S0", d["S0"])
    o, S = oracle.gdn2_recurrent(*(x[n] for n in NAMES), S0=S0)
    return float(np.sum(o * dO) + np.sum(S * dS))


@pytest.mark.parametrize("seed", range(3))
def test_gradients_match_central_differences(seed):
    d = gdn2_inputs(1, 2, 7, 4, 3, alpha_mu=1.0, alpha_sigma=1.0, seed=seed, dtype="f32", s0_std=0.5)
    rng = np.random.default_rng(100 + seed)
    dO = rng.standard_normal((1, 2, 7, 3))
    dS = rng.standard_normal((1, 2, 4, 3))
    g = gdn2_grad(*(d[n] for n in NAMES), d["S0"], dO, dS)
    eps = 1e-6
    for name, key in list(zip(NAMES, ("dq", "dk", "dv", "dalpha", "db", "dw"))) + [("S0", "dS0")]:
        base = d[name]
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = base.copy(), base.copy()
            xp[idx] += eps
            xm[idx] -= eps
            fd = (_loss(d, dO, dS, **{name: xp}) - _loss(d, dO, dS, **{name: xm})) / (2 * eps)
            assert abs(fd - g[key][idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, g[key][idx])


def test_linear_attention_closed_form_gradients():
    """alpha = 1, b = 0, w = 1: o_t = q_t (S0 + sum_{s<=t} k_s^T v_s), so
    dq_t = dO_t S_t^T, dv_s = sum_{t>=s} (q_t . k_s) dO_t + k_s dS_T, dk_s = sum_{t>=s}
    (dO_t . v_s) q_t + dS_T v_s^T, dS0 = sum_t q_t^T dO_t + dS_T."""
    rng = np.random.default_rng(7)
    B, H, T, dk, dv = 1, 2, 6, 3, 4
    q, k = rng.standard_normal((B, H, T, dk)), rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    S0 = rng.standard_normal((B, H, dk, dv))
    dO, dS = rng.standard_normal((B, H, T, dv)), rng.standard_normal((B, H, dk, dv))
    g = gdn2_grad(q, k, v, np.ones((B, H, T, dk)), np.zeros((B, H, T, dk)), np.ones((B, H, T, dv)), S0, dO, dS)
    S = S0[:, :, None] + np.cumsum(np.einsum("bhti,bhtj->bhtij", k, v), axis=2)   # S_t
    dq = np.einsum("bhtj,bhtij->bhti", dO, S)
    mask = np.triu(np.ones((T, T)))                                        # [s, t]: t >= s
    qk = np.einsum("bhti,bhsi->bhst", q, k) * mask
    dv_ = np.einsum("bhst,bhtj->bhsj", qk, dO) + np.einsum("bhsi,bhij->bhsj", k, dS)
    dov = np.einsum("bhtj,bhsj->bhst", dO, v) * mask
    dk_ = np.einsum("bhst,bhti->bhsi", dov, q) + np.einsum("bhij,bhsj->bhsi", dS, v)
    dS0 = np.einsum("bhti,bhtj->bhij", q, dO) + dS
    for key, ref in (("dq", dq), ("dv", dv_), ("dk", dk_), ("dS0", dS0)):
        assert np.allclose(g[key], ref, rtol=0, atol=1e-12), key


def test_decay_gradient_closed_form_one_step():
    """T = 1, S0 given, b = 0: o = q (Diag(alpha) S0 + k^T (w*v)), so
    dalpha_j = sum_c (q_j dO_c) S0[j, c] and dw_c = dO_c v_c (q . k)."""
    rng = np.random.default_rng(8)
    q, k = rng.standard_normal((1, 1, 1, 3)), rng.standard_normal((1, 1, 1, 3))
    v, w = rng.standard_normal((1, 1, 1, 2)), rng.uniform(0.1, 1, (1, 1, 1, 2))
    alpha = rng.uniform(0.1, 1, (1, 1, 1, 3))
    S0 = rng.standard_normal((1, 1, 3, 2))
    dO = rng.standard_normal((1, 1, 1, 2))
    g = gdn2_grad(q, k, v, alpha, np.zeros_like(alpha), w, S0, dO)
    da = np.einsum("j,c,jc->j", q[0, 0, 0], dO[0, 0, 0], S0[0, 0])
    dw = dO[0, 0, 0] * v[0, 0, 0] * np.dot(q[0, 0, 0], k[0, 0, 0])
    assert np.allclose(g["dalpha"][0, 0, 0], da, atol=1e-14) and np.allclose(g["dw"][0, 0, 0], dw, atol=1e-14)
