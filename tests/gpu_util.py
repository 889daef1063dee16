"""Helpers for the GPU parity tests: move seeded inputs to the device and
measure errors against the float64 oracle.

Three measures are used side by side:

* ``rel_err`` — max over heads of the relative Frobenius error of a whole
  per-head array (T x d_v outputs, or the d_k x d_v state): the bar of the
  method's tolerance, 1e-4 for float32 inputs and 2e-2 for bfloat16 inputs
  with a float32 state.
* ``token_err`` — max over (b, h, t) of ||o_t - ref_t|| / ||ref_t||, with the
  denominator floored at a tenth of the head's RMS row norm (a row whose
  reference nearly cancels to zero would otherwise turn a normal absolute
  error into a large relative one). It catches one lost or corrupted token
  (relative error 1), which a whole-head norm would dilute by 1/sqrt(T).
* ``elem_err`` — max over elements of |x - ref| / (|ref| + atol), with atol
  1% of the head's largest reference magnitude: an elementwise bound, used
  for the float32 paths, whose whole-head errors (about 2e-7) also meet a
  bar ten times tighter than the method's (``F32_TIGHT``).
"""
import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}
# per-token bound (rows of o): bf16 outputs are rounded to 8 significant bits
# on their own, so a row carries about 2^-9 relative error before any
# arithmetic error
TOKEN_TOL = {"f32": 1e-4, "bf16": 5e-2}
# float32 inputs: elementwise |x - ref| <= 1e-4 * (|ref| + 1e-2 * max|ref|), and
# the whole-head error at a tenth of the method's bar
ELEM_TOL_F32 = 1e-4
ELEM_ATOL_FRAC = 1e-2
F32_TIGHT = 1e-5
TOKEN_FLOOR = 0.1


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def dev(x, dtype="f32"):
    """float64 numpy array holding dtype-representable values -> device tensor (exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.float32)
    return t.to(torch_dtype(dtype)).cuda()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(x, ref, lead=2):
    """max over the leading `lead` axes of ||x - ref||_F / ||ref||_F."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ax = tuple(range(lead, ref.ndim))
    num = np.sqrt(np.sum((x - ref) ** 2, axis=ax))
    den = np.sqrt(np.sum(ref ** 2, axis=ax))
    return float(np.max(num / np.maximum(den, 1e-300)))


def token_err(x, ref, floor=TOKEN_FLOOR):
    """max over (b, h, t) of ||x_t - ref_t|| / max(||ref_t||, floor * rms_h), for
    outputs [B, H, T, d]; rms_h is the root-mean-square row norm of head h."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(x - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    rms = np.sqrt(np.mean(den ** 2, axis=-1, keepdims=True))
    return float(np.max(num / np.maximum(den, np.maximum(floor * rms, 1e-300))))


def elem_err(x, ref, lead=2, atol_frac=ELEM_ATOL_FRAC):
    """max over elements of |x - ref| / (|ref| + atol_frac * max|ref| of the head)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ax = tuple(range(lead, ref.ndim))
    scale = np.max(np.abs(ref), axis=ax, keepdims=True)
    return float(np.max(np.abs(x - ref) / (np.abs(ref) + np.maximum(atol_frac * scale, 1e-300))))


def check_outputs(o, o_ref, S, S_ref, dtype, label, tol=None):
    """Assert the three measures for an (o, S_T) pair; returns (err_o, err_S, tok_o)."""
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S)), label
    tol = TOL[dtype] if tol is None else tol
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    to = token_err(o, o_ref)
    msg = f"{label}: err_o={eo:.3e} err_S={es:.3e} tok_o={to:.3e}"
    if dtype == "f32":
        ee_o, ee_s = elem_err(o, o_ref), elem_err(S, S_ref)
        msg += f" elem_o={ee_o:.3e} elem_S={ee_s:.3e}"
    say(msg + f" tol={tol:g}")
    assert eo <= tol and es <= tol, msg
    assert to <= max(TOKEN_TOL[dtype], tol), msg
    if dtype == "f32":
        assert ee_o <= ELEM_TOL_F32 and ee_s <= ELEM_TOL_F32, msg
        assert eo <= min(tol, F32_TIGHT) and es <= min(tol, F32_TIGHT), msg
    return eo, es, to


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
