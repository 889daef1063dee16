"""Gated delta-rule matrix-memory kernels for AMD MI355X — Python binding.

A thin ctypes layer over ``libgdr.so`` (see ``include/gdr.h``): it checks
tensor shapes and dtypes, allocates outputs with torch, and passes raw device
pointers and the current HIP stream to the C entry points. Every step of the
computation runs in the library's HIP kernels; there is no fallback. If the
library has not been built the first call raises. With the environment
variable ``GDR_DEBUG=1`` the binding loads ``libgdr_debug.so`` instead: the
same kernels, with every entry point first checking on the GPU that its inputs
are finite and its decays lie in (0, 1] (a :class:`GdrError` with status
``GDR_ERR_PRECONDITION`` names the offending arguments).

Entry points (same names as the C ABI):

* :func:`gdr_chunk_fwd` — chunkwise forward of the channel-wise gated delta
  rule ("Muir: Linear Attention with Sensitivity-Allocated Gating and
  Matched-Filter Readout", §2.1 eq.(1), §2.2), one fused kernel.
* :func:`gdr_chunk_fwd_ws` — the same computation as an intra-chunk kernel
  over all chunks plus a chunk scan, through a device workspace
  (:func:`gdr_chunk_workspace_size` bytes).
* :func:`gdr_decode_step` — one recurrent decode step, state updated in place.
* :func:`gdr_mlstm_fwd` — chunkwise forward of the stabilised mLSTM cell
  ("Exponential gates and matrix memory: xLSTM and RWKV-7", §13.4), one
  fused kernel; :func:`gdr_mlstm_fwd_ws` the same as an intra-chunk kernel
  plus a chunk scan through a workspace.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

__all__ = ["gdr_chunk_fwd", "gdr_chunk_fwd_ws", "gdr_chunk_fwd_noalloc", "gdr_muir_chunk_fwd_ws",
           "gdr_chunk_bwd", "gdr_chunk_bwd_workspace_size", "gdr_rwkv7_fwd", "gdr_rwkv7_workspace_size",
           "gdr_rwkv7_decode_step",
           "gdr_muir_decode_step", "gdr_chunk_workspace_size", "gdr_chunk_intra",
           "gdr_chunk_scan", "gdr_mlstm_fwd_ws", "gdr_mlstm_workspace_size", "gdr_decode_step", "gdr_mlstm_fwd", "gdr_version", "lib_path",
           "GdrError", "load_library", "declare"]

_PKG = os.path.dirname(os.path.abspath(__file__))
# GDR_DEBUG=1 selects the debug library: the same kernels, with every entry
# point checking its inputs' values (finite; decays in (0, 1]) on the GPU
# before it enqueues them, and returning GDR_ERR_PRECONDITION otherwise
DEBUG = os.environ.get("GDR_DEBUG", "0") not in ("", "0")
lib_path = os.path.join(_PKG, "libgdr_debug.so" if DEBUG else "libgdr.so")
GDR_ERR_PRECONDITION = -10

GDR_F32, GDR_BF16 = 0, 1
_lib = None


class GdrError(RuntimeError):
    """A libgdr entry point returned a negative status."""

    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def load_library():
    """Load libgdr.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RuntimeError(
            f"{lib_path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "(or `python matrix_memory_rnn_amd/build.py`); there is no fallback implementation")
    # torch's HIP runtime is loaded first, so that the library binds to the
    # same runtime instance instead of initialising a second one (which then
    # may see no device)
    import torch  # noqa: F401
    _lib = declare(ctypes.CDLL(lib_path))
    return _lib


def declare(lib):
    """Set the argument and result types of every entry point on a loaded
    libgdr (any of its builds); returns ``lib``."""
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.gdr_chunk_fwd.argtypes = [P] * 9 + [I] * 7 + [P]
    lib.gdr_chunk_fwd.restype = I
    lib.gdr_chunk_workspace_size.argtypes = [I] * 7 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_chunk_workspace_size.restype = I
    lib.gdr_chunk_fwd_ws.argtypes = [P] * 9 + [I] * 7 + [P, ctypes.c_size_t, P]
    lib.gdr_chunk_fwd_ws.restype = I
    lib.gdr_chunk_intra.argtypes = [P] * 6 + [I] * 7 + [P, ctypes.c_size_t, P]
    lib.gdr_chunk_intra.restype = I
    lib.gdr_chunk_fwd_noalloc.argtypes = [P] * 9 + [I] * 7 + [P]
    lib.gdr_chunk_fwd_noalloc.restype = I
    lib.gdr_chunk_scan.argtypes = [P, ctypes.c_size_t, P, P, P] + [I] * 7 + [P]
    lib.gdr_chunk_scan.restype = I
    lib.gdr_muir_chunk_fwd_ws.argtypes = [P] * 12 + [I] * 7 + [P, ctypes.c_size_t, P]
    lib.gdr_muir_chunk_fwd_ws.restype = I
    lib.gdr_muir_decode_step.argtypes = [P] * 11 + [I] * 5 + [P]
    lib.gdr_muir_decode_step.restype = I
    lib.gdr_chunk_bwd_workspace_size.argtypes = [I] * 7 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_chunk_bwd_workspace_size.restype = I
    lib.gdr_chunk_bwd.argtypes = [P] * 16 + [I] * 7 + [P, ctypes.c_size_t, I, P]
    lib.gdr_chunk_bwd.restype = I
    lib.gdr_rwkv7_workspace_size.argtypes = [I] * 6 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_rwkv7_workspace_size.restype = I
    lib.gdr_rwkv7_fwd.argtypes = [P] * 9 + [I] * 7 + [P, ctypes.c_size_t, P]
    lib.gdr_rwkv7_fwd.restype = I
    lib.gdr_rwkv7_decode_step.argtypes = [P] * 8 + [I] * 5 + [P]
    lib.gdr_rwkv7_decode_step.restype = I
    lib.gdr_decode_step.argtypes = [P] * 8 + [I] * 5 + [P]
    lib.gdr_decode_step.restype = I
    lib.gdr_mlstm_fwd.argtypes = [P] * 12 + [I] * 7 + [P]
    lib.gdr_mlstm_fwd.restype = I
    lib.gdr_mlstm_workspace_size.argtypes = [I] * 7 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_mlstm_workspace_size.restype = I
    lib.gdr_mlstm_fwd_ws.argtypes = [P] * 12 + [I] * 7 + [P, ctypes.c_size_t, P]
    lib.gdr_mlstm_fwd_ws.restype = I
    lib.gdr_status_string.argtypes = [I]
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_version.argtypes = []
    lib.gdr_version.restype = I
    lib.gdr_debug_build.argtypes = []
    lib.gdr_debug_build.restype = I
    lib.gdr_debug_violation.argtypes = []
    lib.gdr_debug_violation.restype = ctypes.c_char_p
    return lib


def gdr_version() -> int:
    return load_library().gdr_version()


def _check(fn, status):
    if status != 0:
        lib = load_library()
        text = lib.gdr_status_string(status).decode()
        if status == GDR_ERR_PRECONDITION:
            text += f" [{lib.gdr_debug_violation().decode()}]"
        raise GdrError(fn, status, text)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDR_BF16
    if t.dtype == torch.float32:
        return GDR_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _alloc_on(stream):
    """Context in which this binding allocates outputs and workspaces: the
    launch stream when one is given, so torch's caching allocator ties the
    memory to the stream the kernels use (a block freed after the call is not
    handed to another stream while those kernels may still run)."""
    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _req(t, name, shape, dtype, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device or not t.is_cuda:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _chunk_args(q, k, v, alpha, b, w, S0, o, S_out, return_state, stream=None):
    import torch
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, d in (("q", q, dk), ("k", k, dk), ("alpha", alpha, dk), ("b", b, dk),
                       ("v", v, dv), ("w", w, dv)):
        _req(t, name, (B, H, T, d), dt, dev)
    if S0 is not None:
        _req(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    with _alloc_on(stream):
        if o is None:
            o = torch.empty((B, H, T, dv), dtype=dt, device=dev)
        if S_out is None and return_state:
            S_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _req(o, "o", (B, H, T, dv), dt, dev)
    if S_out is not None:
        _req(S_out, "S_out", (B, H, dk, dv), torch.float32, dev)
    return (B, H, T, dk, dv), o, S_out


def gdr_chunk_fwd(q, k, v, alpha, b, w, S0=None, *, chunk=64, o=None, S_out=None,
                  return_state=True, stream=None):
    """Chunkwise gated delta rule over whole sequences (single fused kernel).

    q, k, alpha, b: ``[B,H,T,dk]``; v, w: ``[B,H,T,dv]`` (bfloat16 or float32,
    all the same dtype, on one GPU). S0: ``[B,H,dk,dv]`` float32 or None (zero
    state). Returns ``(o, S_T)`` with o ``[B,H,T,dv]`` in the input dtype and
    S_T float32 (None if ``return_state`` is False). ``S_out`` may be S0 for
    an in-place state update.
    """
    (B, H, T, dk, dv), o, S_out = _chunk_args(q, k, v, alpha, b, w, S0, o, S_out, return_state,
                                                stream)
    lib = load_library()
    st = lib.gdr_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(S0),
                           _ptr(o), _ptr(S_out), B, H, T, dk, dv, int(chunk), _dtype_code(q),
                           _stream(stream))
    _check("gdr_chunk_fwd", st)
    return o, S_out


def gdr_chunk_workspace_size(B, H, T, dk, dv, chunk=64, dtype=None) -> int:
    """Bytes of workspace :func:`gdr_chunk_fwd_ws` needs (dtype: torch dtype, default bf16)."""
    import torch
    code = GDR_BF16 if dtype in (None, torch.bfloat16) else GDR_F32 if dtype == torch.float32 else -1
    n = ctypes.c_size_t(0)
    st = load_library().gdr_chunk_workspace_size(int(B), int(H), int(T), int(dk), int(dv), int(chunk),
                                                 code, ctypes.byref(n))
    _check("gdr_chunk_workspace_size", st)
    return int(n.value)


def gdr_chunk_fwd_ws(q, k, v, alpha, b, w, S0=None, *, chunk=64, o=None, S_out=None,
                     workspace=None, return_state=True, stream=None):
    """Chunkwise gated delta rule as two kernels through a device workspace.

    Same arguments and results as :func:`gdr_chunk_fwd`. ``workspace`` is a
    CUDA tensor of at least :func:`gdr_chunk_workspace_size` bytes (any dtype,
    contiguous); if None, one is allocated for this call.
    """
    import torch
    (B, H, T, dk, dv), o, S_out = _chunk_args(q, k, v, alpha, b, w, S0, o, S_out, return_state,
                                                stream)
    need = gdr_chunk_workspace_size(B, H, T, dk, dv, chunk, q.dtype)
    workspace = _workspace(workspace, need, q.device, stream)
    nbytes = workspace.numel() * workspace.element_size()
    lib = load_library()
    st = lib.gdr_chunk_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(S0),
                              _ptr(o), _ptr(S_out), B, H, T, dk, dv, int(chunk), _dtype_code(q),
                              _ptr(workspace), nbytes, _stream(stream))
    _check("gdr_chunk_fwd_ws", st)
    return o, S_out


def gdr_chunk_fwd_noalloc(q, k, v, alpha, b, w, S0=None, *, chunk=64, o, S_out=None, stream=None):
    """:func:`gdr_chunk_fwd_ws` through the library's static scratch array: no
    workspace and no allocation, by the binding or the library, so the caller
    passes ``o`` (and ``S_out`` if wanted). Returns ``(o, S_out)``. Calls that
    may overlap on one GPU share the array and must be ordered."""
    if o is None:
        raise ValueError("gdr_chunk_fwd_noalloc allocates nothing: pass o (and S_out)")
    (B, H, T, dk, dv), o, S_out = _chunk_args(q, k, v, alpha, b, w, S0, o, S_out, False, stream)
    st = load_library().gdr_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w),
                                              _ptr(S0), _ptr(o), _ptr(S_out), B, H, T, dk, dv, int(chunk),
                                              _dtype_code(q), _stream(stream))
    _check("gdr_chunk_fwd_noalloc", st)
    return o, S_out


def gdr_chunk_bwd_workspace_size(B, H, T, dk, dv, chunk=64, dtype=None) -> int:
    """Bytes of workspace :func:`gdr_chunk_bwd` needs (dtype: torch dtype, default bf16)."""
    import torch
    code = GDR_BF16 if dtype in (None, torch.bfloat16) else GDR_F32 if dtype == torch.float32 else -1
    n = ctypes.c_size_t(0)
    st = load_library().gdr_chunk_bwd_workspace_size(int(B), int(H), int(T), int(dk), int(dv), int(chunk),
                                                     code, ctypes.byref(n))
    _check("gdr_chunk_bwd_workspace_size", st)
    return int(n.value)


def gdr_chunk_bwd(q, k, v, alpha, b, w, S0, dO, dS_T=None, *, chunk=64, workspace=None, records_ready=False,
                  want_dS0=True, stream=None):
    """Gradients of the chunkwise forward ("Muir: ...", §4.2 "Custom Backward
    Pass") for output gradient dO ``[B,H,T,dv]`` (input dtype) and optional
    final-state gradient dS_T ``[B,H,dk,dv]`` float32. Returns a dict of
    float32 tensors dq, dk, dv, dalpha, db, dw (shaped like the inputs) and
    dS0 (``[B,H,dk,dv]``, if ``want_dS0``). ``workspace``: at least
    :func:`gdr_chunk_bwd_workspace_size` bytes; ``records_ready`` when its
    leading records were written by the forward for these inputs."""
    import torch
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, d in (("q", q, dk), ("k", k, dk), ("alpha", alpha, dk), ("b", b, dk),
                       ("v", v, dv), ("w", w, dv), ("dO", dO, dv)):
        _req(t, name, (B, H, T, d), dt, dev)
    for name, t in (("S0", S0), ("dS_T", dS_T)):
        if t is not None:
            _req(t, name, (B, H, dk, dv), torch.float32, dev)
    need = gdr_chunk_bwd_workspace_size(B, H, T, dk, dv, chunk, dt)
    workspace = _workspace(workspace, need, dev, stream)
    with _alloc_on(stream):
        g = {n: torch.empty((B, H, T, d), dtype=torch.float32, device=dev)
             for n, d in (("dq", dk), ("dk", dk), ("dv", dv), ("dalpha", dk), ("db", dk), ("dw", dv))}
        g["dS0"] = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_dS0 else None
    st = load_library().gdr_chunk_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(S0), _ptr(dO), _ptr(dS_T),
        _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dalpha"]), _ptr(g["db"]), _ptr(g["dw"]),
        _ptr(g["dS0"]), B, H, T, dk, dv, int(chunk), _dtype_code(q), _ptr(workspace),
        workspace.numel() * workspace.element_size(), int(bool(records_ready)), _stream(stream))
    _check("gdr_chunk_bwd", st)
    return g


def gdr_rwkv7_workspace_size(B, H, T, dk, dv, chunk=32) -> int:
    """Bytes of workspace :func:`gdr_rwkv7_fwd` needs (float32 records)."""
    n = ctypes.c_size_t(0)
    st = load_library().gdr_rwkv7_workspace_size(int(B), int(H), int(T), int(dk), int(dv), int(chunk),
                                                 ctypes.byref(n))
    _check("gdr_rwkv7_workspace_size", st)
    return int(n.value)


def gdr_rwkv7_fwd(q, w, a, c, kw, u, S0=None, *, chunk=32, o=None, S_out=None, workspace=None,
                  return_state=True, stream=None):
    """RWKV-7 generalized delta rule over whole sequences ("Exponential gates and
    matrix memory: xLSTM and RWKV-7", §13.3): q, w, a, kw ``[B,H,T,dk]`` and u
    ``[B,H,T,dv]`` (bf16 or fp32), c ``[B,H,T]`` float32, S0 ``[B,H,dk,dv]``
    float32 or None. Returns ``(o, S_T)``."""
    import torch
    B, H, T, dk = q.shape
    dv = u.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, d in (("q", q, dk), ("w", w, dk), ("a", a, dk), ("kw", kw, dk), ("u", u, dv)):
        _req(t, name, (B, H, T, d), dt, dev)
    _req(c, "c", (B, H, T), torch.float32, dev)
    if S0 is not None:
        _req(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    with _alloc_on(stream):
        if o is None:
            o = torch.empty((B, H, T, dv), dtype=dt, device=dev)
        if S_out is None and return_state:
            S_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    workspace = _workspace(workspace, gdr_rwkv7_workspace_size(B, H, T, dk, dv, chunk), dev, stream)
    st = load_library().gdr_rwkv7_fwd(_ptr(q), _ptr(w), _ptr(a), _ptr(c), _ptr(kw), _ptr(u), _ptr(S0), _ptr(o),
                                      _ptr(S_out), B, H, T, dk, dv, int(chunk), _dtype_code(q), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream))
    _check("gdr_rwkv7_fwd", st)
    return o, S_out


def gdr_rwkv7_decode_step(q, w, a, c, kw, u, S, *, o=None, stream=None):
    """One RWKV-7 token for N sequences: q, w, a, kw ``[N,H,dk]``, u ``[N,H,dv]``,
    c ``[N,H]`` float32, S ``[N,H,dk,dv]`` float32 updated in place. Returns o."""
    import torch
    N, H, dk = q.shape
    dv = u.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, d in (("q", q, dk), ("w", w, dk), ("a", a, dk), ("kw", kw, dk), ("u", u, dv)):
        _req(t, name, (N, H, d), dt, dev)
    _req(c, "c", (N, H), torch.float32, dev)
    _req(S, "S", (N, H, dk, dv), torch.float32, dev)
    if o is None:
        with _alloc_on(stream):
            o = torch.empty((N, H, dv), dtype=dt, device=dev)
    st = load_library().gdr_rwkv7_decode_step(_ptr(q), _ptr(w), _ptr(a), _ptr(c), _ptr(kw), _ptr(u), _ptr(S),
                                              _ptr(o), N, H, dk, dv, _dtype_code(q), _stream(stream))
    _check("gdr_rwkv7_decode_step", st)
    return o


def _workspace(workspace, need, device, stream=None):
    import torch
    if workspace is None:
        with _alloc_on(stream):
            return torch.empty(need, dtype=torch.uint8, device=device)
    if not (isinstance(workspace, torch.Tensor) and workspace.device == device and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    return workspace


def gdr_chunk_intra(q, k, v, alpha, b, w, *, chunk=64, workspace=None, stream=None):
    """First kernel of :func:`gdr_chunk_fwd_ws`: fills and returns the workspace."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    for name, t, d in (("q", q, dk), ("k", k, dk), ("alpha", alpha, dk), ("b", b, dk),
                       ("v", v, dv), ("w", w, dv)):
        _req(t, name, (B, H, T, d), q.dtype, q.device)
    need = gdr_chunk_workspace_size(B, H, T, dk, dv, chunk, q.dtype)
    workspace = _workspace(workspace, need, q.device, stream)
    st = load_library().gdr_chunk_intra(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w),
                                        B, H, T, dk, dv, int(chunk), _dtype_code(q), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("gdr_chunk_intra", st)
    return workspace


def gdr_chunk_scan(workspace, S0, o, S_out, *, B, H, T, dk, dv, chunk=64, stream=None):
    """Second kernel of :func:`gdr_chunk_fwd_ws`: o ``[B,H,T,dv]`` (input dtype) and
    optional S0 / S_out ``[B,H,dk,dv]`` float32 from a workspace filled by
    :func:`gdr_chunk_intra` with the same sizes."""
    import torch
    _req(o, "o", (B, H, T, dv), o.dtype, o.device)
    for name, t in (("S0", S0), ("S_out", S_out)):
        if t is not None:
            _req(t, name, (B, H, dk, dv), torch.float32, o.device)
    st = load_library().gdr_chunk_scan(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _ptr(S0), _ptr(o), _ptr(S_out), B, H, T, dk, dv, int(chunk),
                                       _dtype_code(o), _stream(stream))
    _check("gdr_chunk_scan", st)
    return o, S_out


def gdr_decode_step(q, k, v, alpha, b, w, S, *, o=None, stream=None):
    """One decode step for N sequences: q, k, alpha, b ``[N,H,dk]``; v, w ``[N,H,dv]``;
    S ``[N,H,dk,dv]`` float32, updated in place. Returns o ``[N,H,dv]``."""
    import torch
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, d in (("q", q, dk), ("k", k, dk), ("alpha", alpha, dk), ("b", b, dk),
                       ("v", v, dv), ("w", w, dv)):
        _req(t, name, (N, H, d), dt, dev)
    _req(S, "S", (N, H, dk, dv), torch.float32, dev)
    if o is None:
        with _alloc_on(stream):
            o = torch.empty((N, H, dv), dtype=dt, device=dev)
    _req(o, "o", (N, H, dv), dt, dev)
    lib = load_library()
    st = lib.gdr_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(S),
                             _ptr(o), N, H, dk, dv, _dtype_code(q), _stream(stream))
    _check("gdr_decode_step", st)
    return o


def _muir_params(q, z_q, a_log, gamma_stat, H, dk, lead):
    import torch
    if z_q is not None:
        _req(z_q, "z_q", tuple(lead) + (dk,), q.dtype, q.device)
    _req(a_log, "a_log", (H,), torch.float32, q.device)
    if gamma_stat is not None:
        _req(gamma_stat, "gamma_stat", (H, dk), torch.float32, q.device)


def gdr_muir_chunk_fwd_ws(q, k, v, z_f, z_b, z_w, a_log, z_q=None, gamma_stat=None, S0=None, *, chunk=64,
                          o=None, S_out=None, workspace=None, return_state=True, stream=None):
    """Chunkwise forward with the Muir gate prologue folded into the kernel:
    z_f, z_b ``[B,H,T,dk]`` and z_w ``[B,H,T,dv]`` are the decay, erase and
    write logits, z_q ``[B,H,T,dk]`` (or None) the query-gain logits, a_log
    ``[H]`` and gamma_stat ``[H,dk]`` (or None) float32 per-head parameters
    ("Muir: ...", §2.1, §4.1 eq.(8)-(9)). Otherwise as :func:`gdr_chunk_fwd_ws`."""
    (B, H, T, dk, dv), o, S_out = _chunk_args(q, k, v, z_f, z_b, z_w, S0, o, S_out, return_state, stream)
    _muir_params(q, z_q, a_log, gamma_stat, H, dk, (B, H, T))
    need = gdr_chunk_workspace_size(B, H, T, dk, dv, chunk, q.dtype)
    workspace = _workspace(workspace, need, q.device, stream)
    st = load_library().gdr_muir_chunk_fwd_ws(
        _ptr(q), _ptr(k), _ptr(v), _ptr(z_f), _ptr(z_b), _ptr(z_w), _ptr(z_q), _ptr(a_log), _ptr(gamma_stat),
        _ptr(S0), _ptr(o), _ptr(S_out), B, H, T, dk, dv, int(chunk), _dtype_code(q), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("gdr_muir_chunk_fwd_ws", st)
    return o, S_out


def gdr_muir_decode_step(q, k, v, z_f, z_b, z_w, a_log, S, z_q=None, gamma_stat=None, *, o=None, stream=None):
    """One decode step with the Muir gate prologue (logits as in
    :func:`gdr_muir_chunk_fwd_ws`, shapes ``[N,H,d]``); S updated in place."""
    import torch
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for name, t, d in (("q", q, dk), ("k", k, dk), ("z_f", z_f, dk), ("z_b", z_b, dk),
                       ("v", v, dv), ("z_w", z_w, dv)):
        _req(t, name, (N, H, d), dt, dev)
    _req(S, "S", (N, H, dk, dv), torch.float32, dev)
    _muir_params(q, z_q, a_log, gamma_stat, H, dk, (N, H))
    if o is None:
        with _alloc_on(stream):
            o = torch.empty((N, H, dv), dtype=dt, device=dev)
    _req(o, "o", (N, H, dv), dt, dev)
    st = load_library().gdr_muir_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(z_f), _ptr(z_b), _ptr(z_w), _ptr(z_q), _ptr(a_log), _ptr(gamma_stat),
        _ptr(S), _ptr(o), N, H, dk, dv, _dtype_code(q), _stream(stream))
    _check("gdr_muir_decode_step", st)
    return o


def _mlstm_args(q, k, v, i_tilde, f_tilde, C0, n0, m0, h, C_out, n_out, m_out, return_state,
                stream=None):
    import torch
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    _req(q, "q", (B, H, T, dk), dt, dev)
    _req(k, "k", (B, H, T, dk), dt, dev)
    _req(v, "v", (B, H, T, dv), dt, dev)
    _req(i_tilde, "i_tilde", (B, H, T), torch.float32, dev)
    _req(f_tilde, "f_tilde", (B, H, T), torch.float32, dev)
    if (C0 is None) != (n0 is None) or (C0 is None) != (m0 is None):
        raise ValueError("pass all of C0, n0, m0 or none of them")
    if C0 is not None:
        _req(C0, "C0", (B, H, dk, dv), torch.float32, dev)
        _req(n0, "n0", (B, H, dk), torch.float32, dev)
        _req(m0, "m0", (B, H), torch.float32, dev)
    with _alloc_on(stream):
        if h is None:
            h = torch.empty((B, H, T, dv), dtype=dt, device=dev)
        if return_state and C_out is None:
            C_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
            n_out = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
            m_out = torch.empty((B, H), dtype=torch.float32, device=dev)
    _req(h, "h", (B, H, T, dv), dt, dev)
    return (B, H, T, dk, dv), h, C_out, n_out, m_out


def gdr_mlstm_fwd(q, k, v, i_tilde, f_tilde, C0=None, n0=None, m0=None, *, chunk=64, h=None,
                  C_out=None, n_out=None, m_out=None, return_state=True, stream=None):
    """Stabilised mLSTM forward (one fused kernel). q, k ``[B,H,T,dk]``, v ``[B,H,T,dv]``
    (bf16/fp32); i_tilde, f_tilde ``[B,H,T]`` float32; optional state (C0 ``[B,H,dk,dv]``,
    n0 ``[B,H,dk]``, m0 ``[B,H]``, float32; all or none). Returns
    ``(h, C_T, n_T, m_T)`` (state entries None if ``return_state`` is False)."""
    (B, H, T, dk, dv), h, C_out, n_out, m_out = _mlstm_args(q, k, v, i_tilde, f_tilde, C0, n0, m0, h,
                                                            C_out, n_out, m_out, return_state, stream)
    lib = load_library()
    st = lib.gdr_mlstm_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(i_tilde), _ptr(f_tilde), _ptr(C0),
                           _ptr(n0), _ptr(m0), _ptr(h), _ptr(C_out), _ptr(n_out), _ptr(m_out),
                           B, H, T, dk, dv, int(chunk), _dtype_code(q), _stream(stream))
    _check("gdr_mlstm_fwd", st)
    return h, C_out, n_out, m_out


def gdr_mlstm_workspace_size(B, H, T, dk, dv, chunk=64, dtype=None) -> int:
    """Bytes of workspace :func:`gdr_mlstm_fwd_ws` needs (dtype: torch dtype, default bf16)."""
    import torch
    code = GDR_BF16 if dtype in (None, torch.bfloat16) else GDR_F32 if dtype == torch.float32 else -1
    n = ctypes.c_size_t(0)
    st = load_library().gdr_mlstm_workspace_size(int(B), int(H), int(T), int(dk), int(dv), int(chunk),
                                                 code, ctypes.byref(n))
    _check("gdr_mlstm_workspace_size", st)
    return int(n.value)


def gdr_mlstm_fwd_ws(q, k, v, i_tilde, f_tilde, C0=None, n0=None, m0=None, *, chunk=64, h=None,
                     C_out=None, n_out=None, m_out=None, workspace=None, return_state=True,
                     stream=None):
    """Stabilised mLSTM forward as two kernels through a workspace (same
    arguments and results as :func:`gdr_mlstm_fwd`; ``workspace`` as for
    :func:`gdr_chunk_fwd_ws`)."""
    (B, H, T, dk, dv), h, C_out, n_out, m_out = _mlstm_args(q, k, v, i_tilde, f_tilde, C0, n0, m0, h,
                                                            C_out, n_out, m_out, return_state, stream)
    need = gdr_mlstm_workspace_size(B, H, T, dk, dv, chunk, q.dtype)
    workspace = _workspace(workspace, need, q.device, stream)
    lib = load_library()
    st = lib.gdr_mlstm_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(i_tilde), _ptr(f_tilde), _ptr(C0),
                              _ptr(n0), _ptr(m0), _ptr(h), _ptr(C_out), _ptr(n_out), _ptr(m_out),
                              B, H, T, dk, dv, int(chunk), _dtype_code(q), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    _check("gdr_mlstm_fwd_ws", st)
    return h, C_out, n_out, m_out
