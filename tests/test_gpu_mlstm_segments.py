"""The segmented wide mLSTM scan (HIP, gfx950) against the float64 oracle.

With few (b, h, 64-column tile) workgroups and at least 32 chunks of 64, the
two-kernel mLSTM forward cuts each head's chunks into a short first segment
and P segments of L chunks. The chunk map of the mLSTM is affine with a
scalar decay ("Exponential gates and matrix memory: xLSTM and RWKV-7", §13.4:
the state is decayed by the forget gate and written by k^T v, with the
max-log stabiliser), so the first segment is scanned beside the end states of
segments 1 .. P-1 from a zero start, and segments 1 .. P are then scanned side
by side, each from the first segment's end state with the maps between
applied. The plan depends on the shapes only; the shapes below take it (bf16,
C = 64, d_k and d_v multiples of 64, B*H*d_v/64 at most 128, at least 32
chunks). The fused entry point never segments, so it serves as the plain scan
to compare with."""
import numpy as np
import pytest

import oracle
from synth import mlstm_inputs
from tests.gpu_util import TOKEN_TOL, TOL, dev, host, rel_err, say, token_err

pytestmark = pytest.mark.gpu

GATES = ("q", "k", "v", "i_tilde", "f_tilde")


def _state(B, H, dk, dv, seed):
    rng = np.random.default_rng(seed)
    C0 = rng.standard_normal((B, H, dk, dv))
    n0 = np.abs(rng.standard_normal((B, H, dk)))
    m0 = rng.uniform(-1, 2, (B, H))
    return C0, n0, m0


def _args(d, state=None):
    t = lambda x: dev(d[x], "bf16")
    g = lambda x: dev(d[x])
    st = (None, None, None) if state is None else tuple(dev(x) for x in state)
    return (t("q"), t("k"), t("v"), g("i_tilde"), g("f_tilde"), *st)


@pytest.mark.parametrize("B,H,T,dk,dv,init", [(1, 2, 64 * 40 + 13, 64, 64, False),     # L0 2, 3 x 13, ragged
                                              (1, 1, 64 * 70, 128, 128, True),        # L0 5, 5 x 13
                                              (2, 2, 64 * 64 + 5, 256, 256, True),    # L0 5, 5 x 12, ragged
                                              (1, 1, 64 * 130 + 37, 64, 64, False)])  # L0 1, 10 x 13, ragged
def test_segmented_mlstm_parity(B, H, T, dk, dv, init):
    import torch
    import matrix_memory_rnn_amd as gdr
    d = mlstm_inputs(B, H, T, dk, dv, seed=T + dk, dtype="bf16")
    state = _state(B, H, dk, dv, T) if init else None
    h, C, n, m = gdr.gdr_mlstm_fwd_ws(*_args(d, state), chunk=64)
    hf, Cf, nf, mf = gdr.gdr_mlstm_fwd(*_args(d, state), chunk=64)
    torch.cuda.synchronize()
    kw = {} if state is None else dict(C0=state[0], n0=state[1], m0=state[2])
    h_ref, C_ref, n_ref, m_ref = oracle.mlstm_stabilized(*(d[x] for x in GATES), **kw)
    h, C, n, m = host(h), host(C), host(n), host(m)
    assert np.all(np.isfinite(h)) and np.all(np.isfinite(C))
    eh, eC, en = rel_err(h, h_ref), rel_err(C, C_ref), rel_err(n, n_ref, lead=2)
    th = token_err(h, h_ref)
    em = float(np.max(np.abs(m - m_ref)))
    label = f"[mseg] B={B} H={H} T={T} dk={dk} dv={dv} init={init}"
    say(f"{label}: err_h={eh:.3e} tok_h={th:.3e} err_C={eC:.3e} err_n={en:.3e} |dm|={em:.2e}")
    assert eh <= TOL["bf16"] and eC <= TOL["bf16"] and en <= TOL["bf16"]
    assert th <= TOKEN_TOL["bf16"]
    assert em <= 1e-4 * max(1.0, np.abs(m_ref).max())
    e1, e2 = rel_err(h, host(hf)), rel_err(C, host(Cf))
    say(f"{label}: segmented vs plain (fused) scan: h {e1:.3e} C {e2:.3e}")
    assert e1 < 1e-2 and e2 < 1e-2


def test_segmented_mlstm_state_in_place():
    """C_out may be C0 on the segmented path too: C0 is read only by the first
    launch and C_out written only by the second, so the in-place call equals
    the one with separate outputs bit for bit."""
    import torch
    import matrix_memory_rnn_amd as gdr
    B, H, T, dk, dv = 1, 2, 64 * 48, 64, 128
    d = mlstm_inputs(B, H, T, dk, dv, seed=41, dtype="bf16")
    C0, n0, m0 = (dev(x) for x in _state(B, H, dk, dv, 41))
    q, k, v, it, ft = _args(d)[:5]
    h1, C1, n1, m1 = gdr.gdr_mlstm_fwd_ws(q, k, v, it, ft, C0, n0, m0, chunk=64)
    Cin = C0.clone()
    n_out, m_out = torch.empty_like(n0), torch.empty_like(m0)
    h2, C2, n2, m2 = gdr.gdr_mlstm_fwd_ws(q, k, v, it, ft, Cin, n0, m0, chunk=64, C_out=Cin, n_out=n_out,
                                          m_out=m_out)
    torch.cuda.synchronize()
    assert C2.data_ptr() == Cin.data_ptr()
    assert torch.equal(h1, h2) and torch.equal(C1, Cin) and torch.equal(n1, n_out) and torch.equal(m1, m_out)


def test_segmented_mlstm_value_column_permutation():
    """Each value column of h and C depends only on the same column of v and
    C0, also across the 64-column tiles of the wide scan: permuting the value
    columns of the inputs permutes the outputs' columns exactly."""
    import torch
    import matrix_memory_rnn_amd as gdr
    B, H, T, dk, dv = 1, 1, 64 * 40, 64, 128
    d = mlstm_inputs(B, H, T, dk, dv, seed=43, dtype="bf16")
    C0, n0, m0 = _state(B, H, dk, dv, 43)
    perm = np.random.default_rng(43).permutation(dv)
    args = lambda vv, cc: (dev(d["q"], "bf16"), dev(d["k"], "bf16"), dev(vv, "bf16"), dev(d["i_tilde"]),
                           dev(d["f_tilde"]), dev(cc), dev(n0), dev(m0))
    h1, C1, n1, m1 = gdr.gdr_mlstm_fwd_ws(*args(d["v"], C0), chunk=64)
    h2, C2, n2, m2 = gdr.gdr_mlstm_fwd_ws(*args(d["v"][..., perm], C0[..., perm]), chunk=64)
    torch.cuda.synchronize()
    p = torch.as_tensor(perm, device=h1.device)
    assert torch.equal(h2, h1.index_select(-1, p)) and torch.equal(C2, C1.index_select(-1, p))
    assert torch.equal(n2, n1) and torch.equal(m2, m1)


def test_segmented_mlstm_without_state_output():
    """Outputs only (no final state pointers): the same h as with the state."""
    import torch
    import matrix_memory_rnn_amd as gdr
    B, H, T, dk, dv = 1, 2, 64 * 36, 128, 64
    d = mlstm_inputs(B, H, T, dk, dv, seed=45, dtype="bf16")
    h1, C1, n1, m1 = gdr.gdr_mlstm_fwd_ws(*_args(d), chunk=64)
    h2 = gdr.gdr_mlstm_fwd_ws(*_args(d), chunk=64, return_state=False)
    if isinstance(h2, tuple):
        h2 = h2[0]
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)
