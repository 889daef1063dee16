"""Float64 oracle of the Muir gate prologue — TEST INFRASTRUCTURE.

Page: "Muir: Linear Attention with Sensitivity-Allocated Gating and
Matched-Filter Readout", §2.1 ("Gated DeltaNet-2" gate parameterisation) and
§4.1 (eq.(9) and the gate list after it; eq.(8), the readout with the
gain-modulated query).

From pre-activation logits the gates are
    log alpha = -exp(a_log) * softplus(z_f),   b = 2 sigmoid(z_b),
    w = sigmoid(z_w),   gamma = gamma_stat * 2 sigmoid(z_q),
and the recurrence is GDN-2's eq.(1) with the readout o_t = (gamma_t * q_t) S_t.
a_log is one number per head, gamma_stat one vector per head.
"""
from __future__ import annotations

import numpy as np

from .gdn2 import gdn2_recurrent, gdn2_step


def softplus(z):
    """log(1 + e^z), without overflow for large z."""
    return np.logaddexp(0.0, np.asarray(z, dtype=np.float64))


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * (1.0 + np.tanh(0.5 * z))


def muir_gates(z_f, z_b, z_w, a_log, z_q=None, gamma_stat=None):
    """Gates from logits. z_f, z_b, z_q: [B,H,T,dk] (or [N,H,dk]); z_w: [...,dv];
    a_log: [H]; gamma_stat: [H, dk] or None (ones); z_q None means z_q = 0.
    Returns (alpha, b, w, gamma) in float64, gamma shaped like z_f."""
    z_f = np.asarray(z_f, dtype=np.float64)
    H = z_f.shape[1]
    extra = z_f.ndim - 3                       # 1 for [B,H,T,d], 0 for [N,H,d]
    rate = np.exp(np.asarray(a_log, dtype=np.float64)).reshape((1, H) + (1,) * (extra + 1))
    alpha = np.exp(-rate * softplus(z_f))
    b = 2.0 * sigmoid(z_b)
    w = sigmoid(z_w)
    gs = np.ones((H, z_f.shape[-1])) if gamma_stat is None else np.asarray(gamma_stat, dtype=np.float64)
    gs = gs.reshape((1, H) + (1,) * extra + (z_f.shape[-1],))
    zq = np.zeros_like(z_f) if z_q is None else np.asarray(z_q, dtype=np.float64)
    gamma = gs * 2.0 * sigmoid(zq)
    return alpha, b, w, gamma


def muir_recurrent(q, k, v, z_f, z_b, z_w, a_log, z_q=None, gamma_stat=None, S0=None):
    """Eq.(8): the GDN-2 recurrence on the gates of ``muir_gates``, read out with
    gamma * q. Returns (o [B,H,T,dv], S_T [B,H,dk,dv])."""
    alpha, b, w, gamma = muir_gates(z_f, z_b, z_w, a_log, z_q, gamma_stat)
    return gdn2_recurrent(gamma * np.asarray(q, dtype=np.float64), k, v, alpha, b, w, S0=S0)


def muir_decode(S, q, k, v, z_f, z_b, z_w, a_log, z_q=None, gamma_stat=None):
    """One decode call on a resident state S [N,H,dk,dv] with inputs [N,H,d]."""
    alpha, b, w, gamma = muir_gates(z_f, z_b, z_w, a_log, z_q, gamma_stat)
    return gdn2_step(np.asarray(S, dtype=np.float64), gamma * np.asarray(q, dtype=np.float64),
                     *(np.asarray(x, dtype=np.float64) for x in (k, v, alpha, b, w)))
