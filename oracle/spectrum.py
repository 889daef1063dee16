"""Spectrum of the diagonal-plus-rank-one transition — TEST INFRASTRUCTURE.

Page: "Exponential gates and matrix memory: xLSTM and RWKV-7", §13.2
(Prop. 13.1), solution to Exercise 13.4 (matrix-determinant lemma, secular
equation, scalar-diagonal spectrum) and §13.3 (reduction to Gated DeltaNet).
These helpers are what the oracle's transition is checked against; they do not
evaluate the recurrence.
"""
from __future__ import annotations

import numpy as np


def generalized_transition(wdiag, c, a):
    """Diag(w) - c a^T a for a row vector a (the page's symmetric generalized transition)."""
    wdiag, a = np.asarray(wdiag, dtype=np.float64), np.asarray(a, dtype=np.float64)
    return np.diag(wdiag) - c * np.outer(a, a)


def scalar_diagonal_spectrum(w0, c, d):
    """Closed form for w = w0*1 and unit a: {w0 - c} union {w0} with multiplicity d-1 (sorted)."""
    return np.sort(np.array([w0 - c] + [w0] * (d - 1), dtype=np.float64))


def secular_residual(lam, wdiag, c, a):
    """f(lambda) = 1 - c * sum_i a_i^2 / (w_i - lambda); zero at eigenvalues off the diagonal entries."""
    wdiag, a = np.asarray(wdiag, dtype=np.float64), np.asarray(a, dtype=np.float64)
    return 1.0 - c * np.sum(a * a / (wdiag - lam))


def symmetrized_transition(k, alpha, b):
    """The GDN-2 transition A = (I - k^T (b*k)) Diag(alpha) = Diag(alpha) - k^T (alpha*b*k)
    is similar, through Diag(sqrt(alpha*b)), to the symmetric Diag(alpha) - c^T c with
    c = sqrt(alpha*b) * k — i.e. to the page's generalized transition with unit direction
    c/|c| and coefficient |c|^2. Returns (Diag(alpha) - c^T c, c)."""
    k, alpha, b = (np.asarray(x, dtype=np.float64) for x in (k, alpha, b))
    c = np.sqrt(alpha * b) * k
    return np.diag(alpha) - np.outer(c, c), c
