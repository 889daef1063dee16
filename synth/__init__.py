"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module draws random numbers and rounds them to the input dtype. It holds
none of the recurrence's arithmetic: the gated delta rule, its chunkwise form
and the mLSTM cell live in ``oracle/`` (CPU, float64) and in the HIP library
(GPU), and neither is imported here.

Input recipe (shapes ``[B, H, T, d]``, head-major, d fastest):

* q, k: draw N(0, 1), apply SiLU, then scale to unit L2 norm over the head
  dimension (the keys and queries of "Muir: Linear Attention with
  Sensitivity-Allocated Gating and Matched-Filter Readout", §2.1, sit on the
  unit sphere after a SiLU), in float64, then round to the input dtype.
  The rounded values are not renormalised.
* v: N(0, 1).
* alpha: sigmoid(N(mu, sigma)) per channel; b, w: sigmoid(N(0, 1)).
* S0 (optional): N(0, s0_std) in float32.
* mLSTM: q, k as above, v ~ N(0, 1), input log-gate ~ N(0, 2) and forget
  logit ~ N(3, 1), both float32.

The second parameter of every N(., .) is a standard deviation. Draw order is
fixed: q, k, v, alpha-logit, b-logit, w-logit, S0 (mLSTM: q, k, v, i, f), all
from ``numpy.random.Generator(PCG64(seed))`` in float64. bfloat16 rounding
is round-to-nearest-even of the float32 value.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "round_to",
    "gdn2_inputs",
    "gdn2_inputs_correlated",
    "decode_inputs",
    "muir_inputs",
    "rwkv7_inputs",
    "mlstm_inputs",
    "CONFIGS",
]


def _bf16_round(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    bits = x32.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = rounded.view(np.float32).copy()
    # NaN/inf pass through unchanged (not produced by these generators).
    special = ~np.isfinite(x32)
    out[special] = x32[special]
    return out


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype`` ("f32" or "bf16"); return them as float64."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32.astype(np.float64)
    if dtype == "bf16":
        return _bf16_round(x32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def _unit_silu(x: np.ndarray) -> np.ndarray:
    s = x * _sigmoid(x)
    return s / np.linalg.norm(s, axis=-1, keepdims=True)


def gdn2_inputs(B, H, T, dk, dv, *, alpha_mu, alpha_sigma, seed=0, dtype="bf16",
                s0_std=None, rng=None):
    """Inputs of the gated delta rule as float64 arrays holding ``dtype`` values.

    Returns a dict with q, k, alpha, b ``[B,H,T,dk]``, v, w ``[B,H,T,dv]`` and
    S0 ``[B,H,dk,dv]`` (float32 values, or None when ``s0_std`` is None).
    """
    g = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    q = _unit_silu(g.standard_normal((B, H, T, dk)))
    k = _unit_silu(g.standard_normal((B, H, T, dk)))
    v = g.standard_normal((B, H, T, dv))
    alpha = _sigmoid(alpha_mu + alpha_sigma * g.standard_normal((B, H, T, dk)))
    b = _sigmoid(g.standard_normal((B, H, T, dk)))
    w = _sigmoid(g.standard_normal((B, H, T, dv)))
    S0 = None
    if s0_std is not None:
        S0 = round_to(s0_std * g.standard_normal((B, H, dk, dv)), "f32")
    out = {name: round_to(x, dtype) for name, x in
           (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("b", b), ("w", w))}
    out["S0"] = S0
    out["dtype"] = dtype
    return out


def gdn2_inputs_correlated(B, H, T, dk, dv, *, n_dirs=4, noise=0.3, b_mu=3.0, b_sigma=0.5,
                           alpha_mu=4.0, alpha_sigma=1.5, seed=0, dtype="bf16", s0_std=None):
    """Inputs whose chunk systems are ill-conditioned, as trained models' are.

    Keys cluster around a few shared directions: per (b, h), ``n_dirs`` unit
    directions are drawn, and key t is the unit vector along direction
    ``idx_t`` (uniform) plus isotropic noise of norm about ``noise``. Erase
    gates sit near the top of the pages' range (0, 2): b = 2*sigmoid(N(b_mu,
    b_sigma)), about 1.9 by default. Repeated, strongly erased keys make the
    unit lower-triangular chunk matrix far from the identity. q, v, alpha, w
    and S0 are drawn as in :func:`gdn2_inputs`.

    Draw order: q, directions, direction indices, key noise, v, alpha-logit,
    b-logit, w-logit, S0, all from ``numpy.random.Generator(PCG64(seed))``.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    q = _unit_silu(g.standard_normal((B, H, T, dk)))
    dirs = g.standard_normal((B, H, n_dirs, dk))
    dirs /= np.linalg.norm(dirs, axis=-1, keepdims=True)
    idx = g.integers(0, n_dirs, size=(B, H, T))
    k = np.take_along_axis(dirs, idx[..., None], axis=2)
    k = k + noise * g.standard_normal((B, H, T, dk)) / np.sqrt(dk)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.standard_normal((B, H, T, dv))
    alpha = _sigmoid(alpha_mu + alpha_sigma * g.standard_normal((B, H, T, dk)))
    b = 2.0 * _sigmoid(b_mu + b_sigma * g.standard_normal((B, H, T, dk)))
    w = _sigmoid(g.standard_normal((B, H, T, dv)))
    S0 = None
    if s0_std is not None:
        S0 = round_to(s0_std * g.standard_normal((B, H, dk, dv)), "f32")
    out = {name: round_to(x, dtype) for name, x in
           (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("b", b), ("w", w))}
    out["S0"] = S0
    out["dtype"] = dtype
    return out


def decode_inputs(N, H, dk, dv, *, step, alpha_mu=4.0, alpha_sigma=1.5, seed=0,
                  dtype="bf16"):
    """One decode step's inputs ``[N,H,d]``, drawn from the seed pair (seed, step)."""
    g = np.random.Generator(np.random.PCG64([seed, step]))
    d = gdn2_inputs(N, H, 1, dk, dv, alpha_mu=alpha_mu, alpha_sigma=alpha_sigma,
                    dtype=dtype, rng=g)
    return {k_: (v_[:, :, 0] if isinstance(v_, np.ndarray) else v_) for k_, v_ in d.items()}


def muir_inputs(B, H, T, dk, dv, *, seed=0, dtype="bf16", zf_mu=-3.0, zf_sigma=1.0, alog_mu=-1.0,
                alog_sigma=0.3, with_zq=True, with_gamma=True, s0_std=None, rng=None):
    """Inputs of the Muir gate prologue: q, k (unit SiLU of N(0,1)), v ~ N(0,1);
    logits z_f ~ N(zf_mu, zf_sigma) (bias included), z_b, z_w, z_q ~ N(0,1)
    (``[B,H,T,d]``, rounded to ``dtype``); a_log ~ N(alog_mu, alog_sigma) per
    head and gamma_stat = exp(N(0, 0.3)) per (head, channel), both float32.
    With the defaults the decays alpha = exp(-exp(a_log) softplus(z_f)) are
    about 0.98 (0.9 to 0.998), like sigmoid(N(4, 1.5)).

    Draw order: q, k, v, z_f, z_b, z_w, z_q, a_log, gamma_stat, S0.
    """
    g = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    q = _unit_silu(g.standard_normal((B, H, T, dk)))
    k = _unit_silu(g.standard_normal((B, H, T, dk)))
    v = g.standard_normal((B, H, T, dv))
    zf = zf_mu + zf_sigma * g.standard_normal((B, H, T, dk))
    zb = g.standard_normal((B, H, T, dk))
    zw = g.standard_normal((B, H, T, dv))
    zq = g.standard_normal((B, H, T, dk))
    alog = alog_mu + alog_sigma * g.standard_normal(H)
    gs = np.exp(0.3 * g.standard_normal((H, dk)))
    S0 = None
    if s0_std is not None:
        S0 = round_to(s0_std * g.standard_normal((B, H, dk, dv)), "f32")
    out = {name: round_to(x, dtype) for name, x in
           (("q", q), ("k", k), ("v", v), ("z_f", zf), ("z_b", zb), ("z_w", zw), ("z_q", zq))}
    if not with_zq:
        out["z_q"] = None
    out["a_log"] = round_to(alog, "f32")
    out["gamma_stat"] = round_to(gs, "f32") if with_gamma else None
    out["S0"] = S0
    out["dtype"] = dtype
    return out


def rwkv7_inputs(B, H, T, dk, dv, *, seed=0, dtype="bf16", w_mu=4.0, w_sigma=1.5, s0_std=None):
    """Inputs of RWKV-7's generalized delta rule: q and the write key kw as the
    GDN-2 keys (unit SiLU of N(0,1)); the removal direction a a unit vector of
    N(0,1); decay w = sigmoid(N(w_mu, w_sigma)) per channel (the GDN-2 decay
    distribution); removal coefficient c = sigmoid(N(0,1)) in (0, 1) per token
    (float32, [B,H,T]); value u ~ N(0,1). Draw order: q, kw, a, u, w-logit,
    c-logit, S0."""
    g = np.random.Generator(np.random.PCG64(seed))
    q = _unit_silu(g.standard_normal((B, H, T, dk)))
    kw = _unit_silu(g.standard_normal((B, H, T, dk)))
    a = g.standard_normal((B, H, T, dk))
    a /= np.linalg.norm(a, axis=-1, keepdims=True)
    u = g.standard_normal((B, H, T, dv))
    w = _sigmoid(w_mu + w_sigma * g.standard_normal((B, H, T, dk)))
    c = _sigmoid(g.standard_normal((B, H, T)))
    S0 = None
    if s0_std is not None:
        S0 = round_to(s0_std * g.standard_normal((B, H, dk, dv)), "f32")
    out = {name: round_to(x, dtype) for name, x in (("q", q), ("w", w), ("a", a), ("kw", kw), ("u", u))}
    out["c"] = round_to(c, "f32")
    out["S0"] = S0
    out["dtype"] = dtype
    return out


def mlstm_inputs(B, H, T, dk, dv, *, seed=0, dtype="bf16", i_sigma=2.0, f_mu=3.0,
                 f_sigma=1.0):
    """mLSTM inputs: q, k ``[B,H,T,dk]``, v ``[B,H,T,dv]`` in ``dtype``; i_tilde, f_tilde ``[B,H,T]`` float32."""
    g = np.random.Generator(np.random.PCG64(seed))
    q = _unit_silu(g.standard_normal((B, H, T, dk)))
    k = _unit_silu(g.standard_normal((B, H, T, dk)))
    v = g.standard_normal((B, H, T, dv))
    i_t = i_sigma * g.standard_normal((B, H, T))
    f_t = f_mu + f_sigma * g.standard_normal((B, H, T))
    return {
        "q": round_to(q, dtype), "k": round_to(k, dtype), "v": round_to(v, dtype),
        "i_tilde": round_to(i_t, "f32"), "f_tilde": round_to(f_t, "f32"),
        "dtype": dtype,
    }


# The five workloads: sizes, chunk length and input distributions.
CONFIGS = {
    "tiny_f32": dict(kind="chunk", B=1, H=2, T=64, dk=16, dv=16, chunk=16,
                     alpha_mu=3.0, alpha_sigma=1.0, dtype="f32", s0_std=None),
    "chunk_4k": dict(kind="chunk", B=4, H=16, T=4096, dk=128, dv=128, chunk=64,
                     alpha_mu=4.0, alpha_sigma=1.5, dtype="bf16", s0_std=None),
    "chunk_32k": dict(kind="chunk", B=1, H=16, T=32768, dk=128, dv=128, chunk=64,
                      alpha_mu=4.0, alpha_sigma=1.5, dtype="bf16", s0_std=0.02),
    "decode": dict(kind="decode", N=256, H=16, dk=128, dv=128, steps=1024,
                   alpha_mu=4.0, alpha_sigma=1.5, dtype="bf16"),
    "mlstm_8k": dict(kind="mlstm", B=2, H=8, T=8192, dk=256, dv=256, chunk=64,
                     dtype="bf16"),
}
