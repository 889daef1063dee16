"""Float64 oracle of the channel-wise gated delta rule (GDN-2) — TEST INFRASTRUCTURE.

Page: "Muir: Linear Attention with Sensitivity-Allocated Gating and
Matched-Filter Readout".

Shapes: q, k, alpha, b ``[B,H,T,dk]``; v, w ``[B,H,T,dv]``; S ``[B,H,dk,dv]``.
Vectors are rows; ``k.T @ x`` is the outer product ``k^T x``.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def gdn2_step(S, q, k, v, alpha, b, w):
    """One token of §2.1 eq.(1), batched over leading axes.

    Decay first (S_hat = Diag(alpha) S), then erase along k with the erase-gated
    key k_hat = b*k reading the *decayed* state, then write k^T (w*v); the
    readout o = q S uses the state after the write.
    Shapes: S [..., dk, dv]; q, k, alpha, b [..., dk]; v, w [..., dv].
    Returns (o [..., dv], S_new [..., dk, dv]).
    """
    S_hat = alpha[..., :, None] * S
    k_hat = b * k
    v_hat = w * v
    read = np.einsum("...i,...ij->...j", k_hat, S_hat)          # k_hat S_hat
    S_new = S_hat - k[..., :, None] * read[..., None, :] + k[..., :, None] * v_hat[..., None, :]
    o = np.einsum("...i,...ij->...j", q, S_new)
    return o, S_new


def gdn2_recurrent(q, k, v, alpha, b, w, S0=None):
    """Sequential evaluation of §2.1 eq.(1) over t = 1..T.

    Returns (o [B,H,T,dv], S_T [B,H,dk,dv]). ``S0=None`` means a zero state.
    """
    q, k, v, alpha, b, w = map(_f64, (q, k, v, alpha, b, w))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, H, T, dv))
    for t in range(T):
        o[:, :, t], S = gdn2_step(S, q[:, :, t], k[:, :, t], v[:, :, t],
                                  alpha[:, :, t], b[:, :, t], w[:, :, t])
    return o, S


def gdn2_decode(S, q, k, v, alpha, b, w):
    """One decode call: the eq.(1) step applied to a resident state ``S [N,H,dk,dv]``."""
    return gdn2_step(_f64(S), *map(_f64, (q, k, v, alpha, b, w)))


def gdn2_transition(k, alpha, b):
    """Materialised transition A_t = (I - k^T (b*k)) Diag(alpha) of §2.1 eq.(1), shape [..., dk, dk]."""
    k, alpha, b = map(_f64, (k, alpha, b))
    dk = k.shape[-1]
    erase = np.eye(dk) - k[..., :, None] * (b * k)[..., None, :]
    return erase * alpha[..., None, :]          # right-multiplying by Diag(alpha) scales columns


def gdn2_materialized(q, k, v, alpha, b, w, S0=None):
    """Same recurrence with explicit dk x dk transition matrices: S_t = A_t S_{t-1} + k_t^T (w_t*v_t)."""
    q, k, v, alpha, b, w = map(_f64, (q, k, v, alpha, b, w))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, H, T, dv))
    for t in range(T):
        A = gdn2_transition(k[:, :, t], alpha[:, :, t], b[:, :, t])
        S = A @ S + k[:, :, t, :, None] * (w[:, :, t] * v[:, :, t])[:, :, None, :]
        o[:, :, t] = np.einsum("bhi,bhij->bhj", q[:, :, t], S)
    return o, S


def gdn2_effective_write(q, k, v, alpha, b, w, S0=None):
    """§2.2's GLA form: S_t = Diag(alpha_t) S_{t-1} + k_t^T v_tilde_t with the
    effective write v_tilde_t = w_t*v_t - (b_t*k_t) Diag(alpha_t) S_{t-1}."""
    q, k, v, alpha, b, w = map(_f64, (q, k, v, alpha, b, w))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, H, T, dv))
    for t in range(T):
        decayed = alpha[:, :, t, :, None] * S
        v_tilde = w[:, :, t] * v[:, :, t] - np.einsum("bhi,bhij->bhj", b[:, :, t] * k[:, :, t], decayed)
        S = decayed + k[:, :, t, :, None] * v_tilde[:, :, None, :]
        o[:, :, t] = np.einsum("bhi,bhij->bhj", q[:, :, t], S)
    return o, S


def delta_rule_textbook(q, k, v, beta, S0=None):
    """Plain DeltaNet: one online-gradient step on 0.5*||k_t S - v_t||^2 with step beta_t,
    S <- S - beta_t k_t^T (k_t S - v_t); readout q_t S_t. beta is [B,H,T]."""
    q, k, v, beta = map(_f64, (q, k, v, beta))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, H, T, dv))
    for t in range(T):
        kt = k[:, :, t]
        resid = np.einsum("bhi,bhij->bhj", kt, S) - v[:, :, t]
        S = S - beta[:, :, t, None, None] * kt[..., :, None] * resid[..., None, :]
        o[:, :, t] = np.einsum("bhi,bhij->bhj", q[:, :, t], S)
    return o, S


def gated_deltanet(q, k, v, gamma, beta, S0=None):
    """Scalar-gated DeltaNet: S <- gamma_t (I - beta_t k_t^T k_t) S + beta_t k_t^T v_t.
    gamma, beta are [B,H,T]."""
    q, k, v, gamma, beta = map(_f64, (q, k, v, gamma, beta))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, H, T, dv))
    eye = np.eye(dk)
    for t in range(T):
        kt = k[:, :, t]
        P = eye - beta[:, :, t, None, None] * kt[..., :, None] * kt[..., None, :]
        S = gamma[:, :, t, None, None] * (P @ S) + beta[:, :, t, None, None] * kt[..., :, None] * v[:, :, t, None, :]
        o[:, :, t] = np.einsum("bhi,bhij->bhj", q[:, :, t], S)
    return o, S


def gla_closed_form(q, k, v, alpha, w, S0=None):
    """Gated linear attention (erase gate b = 0), written as an O(T^2) sum:
    o_t = (q_t * pi_t) S0 + sum_{s<=t} <q_t, pi_{t,s} * k_s> (w_s*v_s),
    with pi_t = prod_{r<=t} alpha_r and pi_{t,s} = prod_{r=s+1..t} alpha_r
    (products, never ratios). Also returns S_T = Diag(pi_T) S0 + sum_s (pi_{T,s}*k_s)^T v_hat_s."""
    q, k, v, alpha, w = map(_f64, (q, k, v, alpha, w))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S0 = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0)
    v_hat = w * v
    o = np.zeros((B, H, T, dv))
    for t in range(T):
        pi_t = np.prod(alpha[:, :, : t + 1], axis=2)
        acc = np.einsum("bhi,bhij->bhj", q[:, :, t] * pi_t, S0)
        for s in range(t + 1):
            pi_ts = np.prod(alpha[:, :, s + 1: t + 1], axis=2)      # empty product = 1
            coef = np.sum(q[:, :, t] * pi_ts * k[:, :, s], axis=-1)
            acc = acc + coef[..., None] * v_hat[:, :, s]
        o[:, :, t] = acc
    pi_T = np.prod(alpha, axis=2)
    S_T = pi_T[..., :, None] * S0
    for s in range(T):
        pi_Ts = np.prod(alpha[:, :, s + 1:], axis=2)
        S_T = S_T + (pi_Ts * k[:, :, s])[..., :, None] * v_hat[:, :, s, None, :]
    return o, S_T


def linear_attention_closed_form(q, k, v, S0=None):
    """Linear attention (alpha = 1, b = 0, w = 1): o_t = q_t S0 + sum_{s<=t} (q_t . k_s) v_s."""
    q, k, v = map(_f64, (q, k, v))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S0 = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0)
    scores = np.einsum("bhti,bhsi->bhts", q, k)
    scores = scores * np.tril(np.ones((T, T)))
    o = np.einsum("bhti,bhij->bhtj", q, S0) + np.einsum("bhts,bhsj->bhtj", scores, v)
    S_T = S0 + np.einsum("bhsi,bhsj->bhij", k, v)
    return o, S_T


def bruteforce_exact(q, k, v, alpha, b, w, S0):
    """Exact rational evaluation for one head with explicit transition products:
    S_T = A_T...A_1 S0 + sum_s A_T...A_{s+1} k_s^T v_hat_s, o_t = q_t S_t.

    All inputs are nested lists (or arrays) of numbers convertible to Fraction
    exactly (use dyadic values); q, k, alpha, b: [T][dk], v, w: [T][dv], S0: [dk][dv].
    Returns (o as [T][dv] Fractions, S_T as [dk][dv] Fractions).
    """
    F = Fraction
    T = len(q)
    dk = len(q[0])
    dv = len(v[0])

    def mat(rows):
        return [[F(x) for x in r] for r in rows]

    def mm(X, Y):
        return [[sum((X[i][m] * Y[m][j] for m in range(len(Y))), F(0)) for j in range(len(Y[0]))]
                for i in range(len(X))]

    def add(X, Y):
        return [[X[i][j] + Y[i][j] for j in range(len(X[0]))] for i in range(len(X))]

    def A_of(t):
        kt = [F(x) for x in k[t]]
        bt = [F(x) for x in b[t]]
        at = [F(x) for x in alpha[t]]
        return [[((1 if i == j else 0) - kt[i] * bt[j] * kt[j]) * at[j] for j in range(dk)]
                for i in range(dk)]

    def write_of(s):
        ks = [F(x) for x in k[s]]
        vh = [F(w[s][j]) * F(v[s][j]) for j in range(dv)]
        return [[ks[i] * vh[j] for j in range(dv)] for i in range(dk)]

    A = [A_of(t) for t in range(T)]
    S0f = mat(S0)
    outs = []
    for t in range(T):
        # S_t = A_t ... A_1 S0 + sum_{s<=t} A_t ... A_{s+1} W_s
        P = S0f
        for r in range(t + 1):
            P = mm(A[r], P)
        St = P
        for s in range(t + 1):
            Ws = write_of(s)
            for r in range(s + 1, t + 1):
                Ws = mm(A[r], Ws)
            St = add(St, Ws)
        qt = [[F(x) for x in q[t]]]
        outs.append(mm(qt, St)[0])
        S_last = St
    return outs, S_last


def _pair_decay(alpha_chunk, t, s):
    """pi_{t,s} = product of alpha_r over r = s+1..t inside one chunk (an empty
    product is 1); alpha_chunk is [..., C, dk]."""
    return np.prod(alpha_chunk[..., s + 1: t + 1, :], axis=-2)


def gdn2_chunk_system(k, alpha, b, chunk):
    """The unit lower-triangular chunk matrices T = I + L_strict of the Muir
    page's §4.2 stage (i): (L_strict)_{t,s} = <b_t*k_t, pi_{t,s}*k_s> for t > s
    inside each chunk, with pi_{t,s} the product of alpha over (s, t].

    k, alpha, b: [B, H, T, dk]. Chunks are consecutive runs of ``chunk`` tokens;
    a shorter last chunk gives a smaller matrix. Returns a list over chunks of
    arrays [B, H, C_c, C_c].
    """
    k, alpha, b = map(_f64, (k, alpha, b))
    Tn = k.shape[2]
    out = []
    for c0 in range(0, Tn, chunk):
        kc, ac, bc = k[:, :, c0:c0 + chunk], alpha[:, :, c0:c0 + chunk], b[:, :, c0:c0 + chunk]
        n = kc.shape[2]
        Tm = np.zeros(kc.shape[:2] + (n, n))
        for t in range(n):
            Tm[:, :, t, t] = 1.0
            for s in range(t):
                Tm[:, :, t, s] = np.sum(bc[:, :, t] * kc[:, :, t] * _pair_decay(ac, t, s) * kc[:, :, s], axis=-1)
        out.append(Tm)
    return out


def gdn2_chunkwise(q, k, v, alpha, b, w, S0=None, chunk=64):
    """The chunkwise form of the Muir page (§2.2 and §4.2 eq.(10)), chunk by chunk:
    T [U | Y] = [V_hat | K_hat_pi] (rows w_t*v_t and pi_t*b_t*k_t), then
    O = (Q_pi - M Y) S0 + M U and S_C = (Diag(pi_C) - K_tilde^T Y) S0 + K_tilde^T U,
    with M_{t,s} = <q_t, pi_{t,s}*k_s> (t >= s), (Q_pi)_t = pi_t*q_t and
    K_tilde_s = pi_{C,s}*k_s. The triangular systems are solved with
    numpy.linalg.solve. A shorter last chunk is handled as a chunk of its own
    length. Returns (o [B,H,T,dv], S_T [B,H,dk,dv]).
    """
    q, k, v, alpha, b, w = map(_f64, (q, k, v, alpha, b, w))
    B, H, Tn, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, H, Tn, dv))
    systems = gdn2_chunk_system(k, alpha, b, chunk)
    for ci, c0 in enumerate(range(0, Tn, chunk)):
        sl = slice(c0, c0 + chunk)
        qc, kc, vc, ac, bc, wc = (x[:, :, sl] for x in (q, k, v, alpha, b, w))
        n = qc.shape[2]
        pi = np.cumprod(ac, axis=2)                                  # pi_t, t = 1..n
        M = np.zeros((B, H, n, n))
        for t in range(n):
            for s in range(t + 1):
                M[:, :, t, s] = np.sum(qc[:, :, t] * _pair_decay(ac, t, s) * kc[:, :, s], axis=-1)
        rhs = np.concatenate([wc * vc, pi * bc * kc], axis=-1)       # [V_hat | K_hat_pi]
        Z = np.linalg.solve(systems[ci], rhs)
        U, Y = Z[..., :dv], Z[..., dv:]
        K_t = np.stack([_pair_decay(ac, n - 1, s) * kc[:, :, s] for s in range(n)], axis=2)
        Q_pi = pi * qc
        o[:, :, sl] = (Q_pi - M @ Y) @ S + M @ U
        S = pi[:, :, -1, :, None] * S - np.swapaxes(K_t, -1, -2) @ Y @ S + np.swapaxes(K_t, -1, -2) @ U
    return o, S


def chunk_condition_numbers(k, alpha, b, chunk):
    """2-norm condition number of every chunk matrix T (see gdn2_chunk_system),
    as an array [B, H, N_chunks] (chunks shorter than 2 tokens give 1)."""
    mats = gdn2_chunk_system(k, alpha, b, chunk)
    return np.stack([np.linalg.cond(m) if m.shape[-1] > 1 else np.ones(m.shape[:2]) for m in mats], axis=-1)
