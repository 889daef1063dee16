"""Float64 oracle of RWKV-7's generalized delta rule — TEST INFRASTRUCTURE.

Page: "Exponential gates and matrix memory: xLSTM and RWKV-7", §13.1 (the
generalized transition Diag(w) - c a a^T), §13.3 (RWKV-7 runs it over a stream:
per-channel decay w_t, unit removal direction a_t, removal coefficient c_t,
and a write u_t b_t^T whose key b_t is decoupled from a_t), the solution to
Exercise 13.5 (the recurrence S_t = S_{t-1}(Diag(w_t) - c_t a_t a_t^T) +
u_t b_t^T and its reduction to Gated DeltaNet).

The page's state is S in R^{d_v x d_k}, read as S q. Here, as everywhere in
this library, the state is its transpose S[d_k, d_v], acted on from the left
and read as o = q S (row vectors):
    S_t = (Diag(w_t) - c_t a_t^T a_t) S_{t-1} + kw_t^T u_t,    o_t = q_t S_t,
with kw the write key (the page's b, renamed so it is not confused with
GDN-2's erase gate). w, a, kw, q: [B,H,T,d_k]; u: [B,H,T,d_v]; c: [B,H,T].
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def rwkv7_step(S, q, w, a, c, kw, u):
    """One token: decay and rank-one removal read the previous state, then the
    write; the readout sees the new state. Shapes: S [..., dk, dv]; q, w, a,
    kw [..., dk]; c [...]; u [..., dv]. Returns (o, S_new)."""
    removed = np.einsum("...i,...ij->...j", a, S)                      # a S_{t-1}
    S_new = w[..., :, None] * S - (c[..., None] * a)[..., :, None] * removed[..., None, :] \
        + kw[..., :, None] * u[..., None, :]
    o = np.einsum("...i,...ij->...j", q, S_new)
    return o, S_new


def rwkv7_recurrent(q, w, a, c, kw, u, S0=None):
    """Sequential evaluation over t = 1..T. Returns (o [B,H,T,dv], S_T)."""
    q, w, a, c, kw, u = map(_f64, (q, w, a, c, kw, u))
    B, H, T, dk = q.shape
    dv = u.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, H, T, dv))
    for t in range(T):
        o[:, :, t], S = rwkv7_step(S, q[:, :, t], w[:, :, t], a[:, :, t], c[:, :, t], kw[:, :, t], u[:, :, t])
    return o, S


def rwkv7_decode(S, q, w, a, c, kw, u):
    """One decode call on resident states S [N,H,dk,dv]; inputs [N,H,d], c [N,H]."""
    return rwkv7_step(_f64(S), *map(_f64, (q, w, a, c, kw, u)))


def rwkv7_materialized(q, w, a, c, kw, u, S0=None):
    """The same recurrence with the d_k x d_k transition matrices written out:
    A_t = Diag(w_t) - c_t a_t^T a_t, S_t = A_t S_{t-1} + kw_t^T u_t."""
    q, w, a, c, kw, u = map(_f64, (q, w, a, c, kw, u))
    B, H, T, dk = q.shape
    dv = u.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, H, T, dv))
    for t in range(T):
        A = np.zeros((B, H, dk, dk))
        idx = np.arange(dk)
        A[:, :, idx, idx] = w[:, :, t]
        A -= c[:, :, t, None, None] * a[:, :, t, :, None] * a[:, :, t, None, :]
        S = A @ S + kw[:, :, t, :, None] * u[:, :, t, None, :]
        o[:, :, t] = np.einsum("bhi,bhij->bhj", q[:, :, t], S)
    return o, S
