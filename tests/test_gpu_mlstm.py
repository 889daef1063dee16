"""Parity of gdr_mlstm_fwd (HIP, gfx950) with the float64 stabilised oracle.

The readout h is unique and compared directly. The stabiliser m is the running
max of the xLSTM page in both implementations, so the scaled state (C, n, m)
is compared directly too (m in absolute terms)."""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, mlstm_inputs
from tests.gpu_util import TOL, dev, host, rel_err, say

pytestmark = pytest.mark.gpu


def _run(d, chunk, state=None):
    import matrix_memory_rnn_amd as gdr
    t = lambda x: dev(d[x], d["dtype"])
    g = lambda x: dev(d[x], "f32")
    st = (None, None, None) if state is None else tuple(dev(x) for x in state)
    return gdr.gdr_mlstm_fwd(t("q"), t("k"), t("v"), g("i_tilde"), g("f_tilde"), *st, chunk=chunk)


def _check(d, chunk, label, state=None):
    import torch
    h, C, n, m = _run(d, chunk, state)
    torch.cuda.synchronize()
    kw = {} if state is None else dict(C0=state[0], n0=state[1], m0=state[2])
    h_ref, C_ref, n_ref, m_ref = oracle.mlstm_stabilized(d["q"], d["k"], d["v"], d["i_tilde"],
                                                         d["f_tilde"], **kw)
    eh, eC, en = rel_err(host(h), h_ref), rel_err(host(C), C_ref), rel_err(host(n), n_ref)
    em = float(np.max(np.abs(host(m) - m_ref)))
    tol = TOL[d["dtype"]]
    say(f"[mlstm] {label}: err_h={eh:.3e} err_C={eC:.3e} err_n={en:.3e} |dm|={em:.2e} tol={tol:g}")
    assert eh <= tol and eC <= tol and en <= tol and em <= 1e-4 * max(1.0, np.abs(m_ref).max())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,chunk", [(16, 16, 16), (64, 64, 64), (128, 32, 32), (32, 128, 64)])
def test_mlstm_shapes(dtype, dk, dv, chunk):
    d = mlstm_inputs(2, 2, 2 * chunk + 9, dk, dv, seed=dk + dv, dtype=dtype)
    _check(d, chunk, f"{dtype} dk={dk} dv={dv} C={chunk}")


def test_mlstm_dk256_bf16():
    d = mlstm_inputs(1, 2, 150, 256, 256, seed=2, dtype="bf16")
    _check(d, 64, "bf16 dk=dv=256")


def test_mlstm_with_initial_state_and_large_gates():
    d = mlstm_inputs(2, 2, 100, 64, 64, seed=4, dtype="f32")
    d["i_tilde"][:, :, 30] = 60.0          # one very strong write
    rng = np.random.default_rng(4)
    C0 = rng.standard_normal((2, 2, 64, 64)).astype(np.float32).astype(np.float64)
    n0 = np.abs(rng.standard_normal((2, 2, 64))).astype(np.float32).astype(np.float64)
    m0 = np.array([[0.5, -1.0], [2.0, 0.0]])
    _check(d, 32, "f32 with initial state, i_tilde = 60", state=(C0, n0, m0))


def test_full_size_mlstm_sampled_heads():
    import torch
    c = CONFIGS["mlstm_8k"]
    d = mlstm_inputs(c["B"], c["H"], c["T"], c["dk"], c["dv"], seed=0, dtype=c["dtype"])
    h, C, n, m = _run(d, c["chunk"])
    torch.cuda.synchronize()
    h, C = host(h), host(C)
    for (bi, hi) in [(0, 0), (1, 7)]:
        sl = lambda x: x[bi:bi + 1, hi:hi + 1]
        h_ref, C_ref, _, _ = oracle.mlstm_stabilized(*(sl(d[x]) for x in ("q", "k", "v", "i_tilde", "f_tilde")))
        eh, eC = rel_err(sl(h), h_ref), rel_err(sl(C), C_ref)
        say(f"[mlstm] full-size head (b={bi},h={hi}): err_h={eh:.3e} err_C={eC:.3e}")
        assert eh <= TOL["bf16"] and eC <= TOL["bf16"]
