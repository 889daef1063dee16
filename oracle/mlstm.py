"""Float64 oracle of the xLSTM mLSTM matrix-memory cell — TEST INFRASTRUCTURE.

Page: "Exponential gates and matrix memory: xLSTM and RWKV-7", §13.4 and the
solution to Exercise 13.6 (the log-domain stabilizer).

The cell carries a matrix memory C, a normaliser n and (stabilised form) a
scalar stabiliser m per head. Gates are scalars per token: forget gate
f_t = sigmoid(f_tilde_t) in (0, 1], input gate i_t = exp(i_tilde_t) unbounded.
Orientation as the rest of the oracle: C[dk, dv], written with k^T v and read as
q C (the page writes the transpose, C[dv, dk] written with v k^T, read C q).

Readings where the page's display equations did not survive extraction:
* stabiliser  m_t = max(log f_t + m_{t-1}, i_tilde_t);
* scaled gates f'_t = exp(log f_t + m_{t-1} - m_t), i'_t = exp(i_tilde_t - m_t);
* C_t = f'_t C_{t-1} + i'_t k_t^T v_t,  n_t = f'_t n_{t-1} + i'_t k_t;
* readout h_t = q_t C_t / max(|q_t . n_t|, exp(-m_t)) — the naive form's floor
  of 1 becomes exp(-m_t) in scaled coordinates; the absolute value is the
  xLSTM convention (the page only prints the q = k case, where q.n > 0);
* empty initial state: C_0 = 0, n_0 = 0, m_0 = -inf, so the first write has
  f'_1 = 0 and i'_1 = 1.
No 1/sqrt(d) key scaling and no output gate: the caller may pre-scale.
"""
from __future__ import annotations

import numpy as np


def log_sigmoid(x):
    """log sigmoid(x) = -softplus(-x), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    return -np.logaddexp(0.0, -x)


def mlstm_stabilized(q, k, v, i_tilde, f_tilde, C0=None, n0=None, m0=None):
    """Stabilised mLSTM over t = 1..T.

    q, k [B,H,T,dk]; v [B,H,T,dv]; i_tilde, f_tilde [B,H,T].
    C0 [B,H,dk,dv], n0 [B,H,dk], m0 [B,H]; None means the empty state (m0 = -inf).
    Returns (h [B,H,T,dv], C_T, n_T, m_T).
    """
    q, k, v, i_tilde, f_tilde = (np.asarray(x, dtype=np.float64) for x in (q, k, v, i_tilde, f_tilde))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    C = np.zeros((B, H, dk, dv)) if C0 is None else np.array(C0, dtype=np.float64)
    n = np.zeros((B, H, dk)) if n0 is None else np.array(n0, dtype=np.float64)
    m = np.full((B, H), -np.inf) if m0 is None else np.array(m0, dtype=np.float64)
    logf = log_sigmoid(f_tilde)
    h = np.zeros((B, H, T, dv))
    for t in range(T):
        m_new = np.maximum(logf[:, :, t] + m, i_tilde[:, :, t])
        with np.errstate(invalid="ignore"):
            fp = np.exp(logf[:, :, t] + m - m_new)           # exp(-inf) = 0 on the first write
        fp = np.where(np.isneginf(m), 0.0, fp)
        ip = np.exp(i_tilde[:, :, t] - m_new)
        C = fp[..., None, None] * C + ip[..., None, None] * k[:, :, t, :, None] * v[:, :, t, None, :]
        n = fp[..., None] * n + ip[..., None] * k[:, :, t]
        m = m_new
        num = np.einsum("bhi,bhij->bhj", q[:, :, t], C)
        den = np.maximum(np.abs(np.sum(q[:, :, t] * n, axis=-1)), np.exp(-m))
        h[:, :, t] = num / den[..., None]
    return h, C, n, m


def mlstm_naive(q, k, v, i_tilde, f_tilde):
    """Unstabilised mLSTM from the empty state: C_t = f_t C_{t-1} + exp(i_tilde_t) k^T v,
    n_t = f_t n_{t-1} + exp(i_tilde_t) k, h_t = q C_t / max(|q . n_t|, 1).
    Overflows float64 once exp(i_tilde) exceeds ~1.8e308 (i_tilde > ~709.78)."""
    q, k, v, i_tilde, f_tilde = (np.asarray(x, dtype=np.float64) for x in (q, k, v, i_tilde, f_tilde))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    C = np.zeros((B, H, dk, dv))
    n = np.zeros((B, H, dk))
    f = np.exp(log_sigmoid(f_tilde))
    h = np.zeros((B, H, T, dv))
    with np.errstate(over="ignore", invalid="ignore"):
        ig = np.exp(i_tilde)
        for t in range(T):
            C = f[:, :, t, None, None] * C + ig[:, :, t, None, None] * k[:, :, t, :, None] * v[:, :, t, None, :]
            n = f[:, :, t, None] * n + ig[:, :, t, None] * k[:, :, t]
            num = np.einsum("bhi,bhij->bhj", q[:, :, t], C)
            den = np.maximum(np.abs(np.sum(q[:, :, t] * n, axis=-1)), 1.0)
            h[:, :, t] = num / den[..., None]
    return h, C, n


def mlstm_with_stabilizer(q, k, v, i_tilde, f_tilde, m_seq):
    """The scaled recurrence driven by an arbitrary stabiliser sequence m_seq [B,H,T]
    (empty initial state). With scaled state C_t = exp(-m_t) C_bar_t the readout
    q C_t / max(|q n_t|, exp(-m_t)) equals the naive one whenever nothing overflows:
    the change of variables of Exercise 13.6(b, c) holds for any m, not only the
    running max."""
    q, k, v, i_tilde, f_tilde, m_seq = (np.asarray(x, dtype=np.float64)
                                        for x in (q, k, v, i_tilde, f_tilde, m_seq))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    C = np.zeros((B, H, dk, dv))
    n = np.zeros((B, H, dk))
    logf = log_sigmoid(f_tilde)
    h = np.zeros((B, H, T, dv))
    for t in range(T):
        m_prev = m_seq[:, :, t - 1] if t > 0 else None
        fp = np.zeros((B, H)) if t == 0 else np.exp(logf[:, :, t] + m_prev - m_seq[:, :, t])
        ip = np.exp(i_tilde[:, :, t] - m_seq[:, :, t])
        C = fp[..., None, None] * C + ip[..., None, None] * k[:, :, t, :, None] * v[:, :, t, None, :]
        n = fp[..., None] * n + ip[..., None] * k[:, :, t]
        num = np.einsum("bhi,bhij->bhj", q[:, :, t], C)
        den = np.maximum(np.abs(np.sum(q[:, :, t] * n, axis=-1)), np.exp(-m_seq[:, :, t]))
        h[:, :, t] = num / den[..., None]
    return h


def stabilizer_closed_form(i_tilde, f_tilde, m0=None):
    """Unrolled running max: with F_t = sum_{r<=t} log f_r,
    m_t = max(F_t + m0, max_{s<=t} (F_t - F_s + i_tilde_s)). Returns m [B,H,T]."""
    i_tilde = np.asarray(i_tilde, dtype=np.float64)
    F = np.cumsum(log_sigmoid(f_tilde), axis=-1)
    T = i_tilde.shape[-1]
    m = np.empty_like(i_tilde)
    base = np.full(i_tilde.shape[:-1], -np.inf) if m0 is None else np.asarray(m0, dtype=np.float64)
    for t in range(T):
        cand = F[..., t, None] - F[..., : t + 1] + i_tilde[..., : t + 1]
        m[..., t] = np.maximum(F[..., t] + base, cand.max(axis=-1))
    return m
