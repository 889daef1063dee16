"""The debug library (libgdr_debug.so, GDR_DEBUG defined) on the GPU: with valid
inputs every entry point returns exactly what the release library returns
(same kernels, plus a read-only check before them); an input that breaks a
value rule (non-finite, or a decay outside (0, 1]) makes the entry point return
GDR_ERR_PRECONDITION before any compute kernel runs, so its outputs stay as
they were, and gdr_debug_violation names the argument."""
import ctypes
import os

import numpy as np
import pytest

from synth import gdn2_inputs, mlstm_inputs, muir_inputs, rwkv7_inputs
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DEBUG = os.path.join(ROOT, "matrix_memory_rnn_amd", "libgdr_debug.so")
SENTINEL = 7.0


@pytest.fixture(scope="module")
def libs():
    import matrix_memory_rnn_amd as m
    rel = m.load_library()
    if not os.path.exists(LIB_DEBUG):
        pytest.fail("libgdr_debug.so is not built")
    dbg = m.declare(ctypes.CDLL(LIB_DEBUG))
    assert dbg.gdr_debug_build() == 1 and rel.gdr_debug_build() == 0
    return rel, dbg


@pytest.fixture
def use(libs, monkeypatch):
    """Returns a function that points the binding at the release or the debug
    library for the calls that follow."""
    import matrix_memory_rnn_amd as m

    def pick(which):
        monkeypatch.setattr(m, "_lib", libs[1] if which == "debug" else libs[0])
        return m
    return pick


def _gdn(dtype="bf16", T=100, d=64):
    x = gdn2_inputs(1, 2, T, d, d, alpha_mu=4.0, alpha_sigma=1.5, seed=21, dtype=dtype, s0_std=0.1)
    return {n: (dev(x[n], dtype) if n != "S0" else dev(x[n])) for n in ("q", "k", "v", "alpha", "b", "w", "S0")}


def _rejects(m, fn, name, outs):
    """Runs fn; expects GDR_ERR_PRECONDITION naming `name` and every output
    tensor in `outs` still holding SENTINEL."""
    import torch
    with pytest.raises(m.GdrError) as e:
        fn()
    torch.cuda.synchronize()
    assert e.value.status == m.GDR_ERR_PRECONDITION, str(e.value)
    assert str(e.value).endswith(f"[{name}]"), str(e.value)
    for t in outs:
        assert bool((t == SENTINEL).all()), "an output was written although the call was rejected"
    say(f"[debug] rejected: {e.value}")


def _full(shape, dtype, like):
    import torch
    return torch.full(shape, SENTINEL, dtype=dtype, device=like.device)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_debug_library_matches_release_on_valid_inputs(use, dtype):
    import torch
    x = _gdn(dtype)
    outs = {}
    for which in ("release", "debug"):
        m = use(which)
        o1, S1 = m.gdr_chunk_fwd_ws(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], x["S0"], chunk=32)
        o2, S2 = m.gdr_chunk_fwd(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], x["S0"], chunk=32)
        S = x["S0"].clone()
        o3 = m.gdr_decode_step(*(x[n][:, :, 5].contiguous() for n in ("q", "k", "v", "alpha", "b", "w")), S)
        torch.cuda.synchronize()
        outs[which] = [host(t) for t in (o1, S1, o2, S2, o3, S)]
    for a, b in zip(outs["release"], outs["debug"]):
        assert np.array_equal(a, b)


def test_chunk_entry_points_reject_bad_values(use):
    import torch
    m = use("debug")
    base = _gdn()
    cases = [("alpha", 0.0, "alpha"), ("alpha", 1.5, "alpha"), ("alpha", float("nan"), "alpha"),
             ("v", float("nan"), "v"), ("k", float("inf"), "k"), ("S0", float("-inf"), "S0")]
    for arg, val, name in cases:
        x = {n: t.clone() for n, t in base.items()}
        x[arg].view(-1)[123] = val
        o = _full(x["v"].shape, x["v"].dtype, x["v"])
        S_out = _full(x["S0"].shape, torch.float32, x["v"])
        for fn in (m.gdr_chunk_fwd_ws, m.gdr_chunk_fwd, m.gdr_chunk_fwd_noalloc):
            _rejects(m, lambda: fn(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], x["S0"], chunk=32,
                                   o=o, S_out=S_out), name, [o, S_out])
    # alpha = 1 exactly is inside the domain
    x = {n: t.clone() for n, t in base.items()}
    x["alpha"][:, :, :7] = 1.0
    m.gdr_chunk_fwd_ws(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], x["S0"], chunk=32)
    torch.cuda.synchronize()
    assert m.load_library().gdr_debug_violation().decode() == ""


def test_several_bad_arguments_are_all_named(use):
    m = use("debug")
    x = _gdn()
    x["q"].view(-1)[0] = float("nan")
    x["w"].view(-1)[-1] = float("inf")
    o = _full(x["v"].shape, x["v"].dtype, x["v"])
    _rejects(m, lambda: m.gdr_chunk_fwd_ws(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], x["S0"],
                                           chunk=32, o=o), "q, w", [o])


def test_decode_rejects_a_non_finite_state(use):
    m = use("debug")
    x = _gdn(T=1)
    S = x["S0"].clone()
    S.view(-1)[77] = float("nan")
    step = [x[n][:, :, 0].contiguous() for n in ("q", "k", "v", "alpha", "b", "w")]
    o = _full(step[2].shape, step[2].dtype, step[2])
    _rejects(m, lambda: m.gdr_decode_step(*step, S, o=o), "S", [o])


def test_mlstm_stabiliser_may_be_minus_infinity(use):
    import torch
    m = use("debug")
    d = mlstm_inputs(1, 2, 64, 64, 64, seed=5, dtype="bf16")
    q, k, v = (dev(d[n], "bf16") for n in ("q", "k", "v"))
    it, ft = dev(d["i_tilde"]), dev(d["f_tilde"])
    C0 = torch.zeros(1, 2, 64, 64, device=q.device)
    n0 = torch.zeros(1, 2, 64, device=q.device)
    m0 = torch.full((1, 2), float("-inf"), device=q.device)
    h_dbg = m.gdr_mlstm_fwd(q, k, v, it, ft, C0, n0, m0, chunk=64)[0]
    m_rel = use("release")
    h_rel = m_rel.gdr_mlstm_fwd(q, k, v, it, ft, C0, n0, m0, chunk=64)[0]
    torch.cuda.synchronize()
    assert np.array_equal(host(h_dbg), host(h_rel))
    m = use("debug")
    h = _full(v.shape, v.dtype, v)
    _rejects(m, lambda: m.gdr_mlstm_fwd(q, k, v, it, ft, C0, n0, torch.full_like(m0, float("inf")), h=h,
                                        return_state=False), "m0", [h])
    ft_bad = ft.clone()
    ft_bad[0, 1, 9] = float("nan")
    _rejects(m, lambda: m.gdr_mlstm_fwd_ws(q, k, v, it, ft_bad, h=h, return_state=False), "f_tilde", [h])


def test_rwkv7_rejects_a_zero_decay(use):
    m = use("debug")
    d = rwkv7_inputs(1, 2, 40, 32, 32, seed=6, dtype="bf16", s0_std=0.1)
    x = {n: dev(d[n], "bf16") for n in ("q", "w", "a", "kw", "u")}
    c, S0 = dev(d["c"]), dev(d["S0"])
    x["w"].view(-1)[50] = 0.0
    o = _full(x["u"].shape, x["u"].dtype, x["u"])
    _rejects(m, lambda: m.gdr_rwkv7_fwd(x["q"], x["w"], x["a"], c, x["kw"], x["u"], S0, o=o), "w", [o])
    step = [x[n][:, :, 3].contiguous() for n in ("q", "w", "a")]
    step[1].view(-1)[0] = 1.25
    rest = [x[n][:, :, 3].contiguous() for n in ("kw", "u")]
    o1 = _full(rest[1].shape, rest[1].dtype, rest[1])
    S = S0.clone()
    _rejects(m, lambda: m.gdr_rwkv7_decode_step(*step, c[:, :, 3].contiguous(), *rest, S, o=o1), "w", [o1])


def test_backward_rejects_a_non_finite_output_gradient(use):
    m = use("debug")
    x = _gdn(T=64, d=32)
    dO = x["v"].clone()
    dO.view(-1)[200] = float("nan")
    with pytest.raises(m.GdrError) as e:
        m.gdr_chunk_bwd(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], x["S0"], dO, chunk=32)
    assert e.value.status == m.GDR_ERR_PRECONDITION and str(e.value).endswith("[dO]"), str(e.value)


def test_muir_rejects_a_non_finite_gate_parameter(use):
    m = use("debug")
    d = muir_inputs(1, 2, 64, 32, 32, seed=8, dtype="bf16")
    x = {n: dev(d[n], "bf16") for n in ("q", "k", "v", "z_f", "z_b", "z_w")}
    a_log = dev(d["a_log"]).clone()
    a_log[1] = float("nan")
    o = _full(x["v"].shape, x["v"].dtype, x["v"])
    _rejects(m, lambda: m.gdr_muir_chunk_fwd_ws(x["q"], x["k"], x["v"], x["z_f"], x["z_b"], x["z_w"], a_log,
                                                o=o, return_state=False), "a_log", [o])
