"""Float64 oracle of the gradients of the GDN-2 recurrence — TEST INFRASTRUCTURE.

Page: "Muir: Linear Attention with Sensitivity-Allocated Gating and
Matched-Filter Readout", §2.1 eq.(1) (the forward) and §4.2 "Custom Backward
Pass" (what training needs: gradients of a scalar loss with respect to every
input of the chunk computation and to the initial state).

For a loss J = sum(dO * O) + sum(dS_T * S_T) the gradients are obtained by
reverse-mode differentiation of eq.(1) written step by step in float64 torch
(CPU) — torch.autograd is the library primitive that does the
differentiating; the step is restated here, not imported from the GPU path.
Pinned by central finite differences of ``gdn2_recurrent`` and by closed forms
(tests/test_oracle_grad.py).
"""
from __future__ import annotations

import numpy as np
import torch


def _step(S, q, k, v, alpha, b, w):
    # eq.(1): decay, erase along k reading the decayed state, write, read out
    S_hat = alpha[..., :, None] * S
    read = torch.einsum("...i,...ij->...j", b * k, S_hat)
    S_new = S_hat - k[..., :, None] * read[..., None, :] + k[..., :, None] * (w * v)[..., None, :]
    o = torch.einsum("...i,...ij->...j", q, S_new)
    return o, S_new


def gdn2_grad(q, k, v, alpha, b, w, S0, dO, dS_T=None):
    """Gradients of J = <dO, O> + <dS_T, S_T> for the recurrence of eq.(1).

    Shapes as for ``gdn2_recurrent``; S0 may be None (zero state, no dS0
    returned as zeros). Returns a dict of float64 arrays dq, dk, dv, dalpha,
    db, dw, dS0."""
    t = lambda x: torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)
    q_, k_, v_, a_, b_, w_ = (t(x) for x in (q, k, v, alpha, b, w))
    B, H, T, dk = q_.shape
    dv = v_.shape[-1]
    S0_ = t(np.zeros((B, H, dk, dv)) if S0 is None else S0)
    S = S0_
    outs = []
    for i in range(T):
        o, S = _step(S, q_[:, :, i], k_[:, :, i], v_[:, :, i], a_[:, :, i], b_[:, :, i], w_[:, :, i])
        outs.append(o)
    O = torch.stack(outs, dim=2)
    J = (O * torch.as_tensor(np.asarray(dO, dtype=np.float64))).sum()
    if dS_T is not None:
        J = J + (S * torch.as_tensor(np.asarray(dS_T, dtype=np.float64))).sum()
    J.backward()
    g = lambda x: x.grad.detach().numpy().copy()
    return {"dq": g(q_), "dk": g(k_), "dv": g(v_), "dalpha": g(a_), "db": g(b_), "dw": g(w_), "dS0": g(S0_)}
