"""Parity of the mLSTM entry points (HIP, gfx950) with the float64 stabilised
oracle: gdr_mlstm_fwd (one fused kernel) and gdr_mlstm_fwd_ws (intra-chunk
kernel plus chunk scan through a workspace).

The readout h is unique and compared directly. The stabiliser m is the running
max of the xLSTM page in both implementations, so the scaled state (C, n, m)
is compared directly too (m in absolute terms)."""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, mlstm_inputs
from tests.gpu_util import TOL, dev, host, rel_err, say

pytestmark = pytest.mark.gpu


PATHS = ["fused", "ws"]


def _run(d, chunk, state=None, path="ws"):
    import matrix_memory_rnn_amd as gdr
    t = lambda x: dev(d[x], d["dtype"])
    g = lambda x: dev(d[x], "f32")
    st = (None, None, None) if state is None else tuple(dev(x) for x in state)
    fn = gdr.gdr_mlstm_fwd if path == "fused" else gdr.gdr_mlstm_fwd_ws
    return fn(t("q"), t("k"), t("v"), g("i_tilde"), g("f_tilde"), *st, chunk=chunk)


def _check(d, chunk, label, state=None, path="ws"):
    import torch
    label = f"{path} {label}"
    h, C, n, m = _run(d, chunk, state, path)
    torch.cuda.synchronize()
    kw = {} if state is None else dict(C0=state[0], n0=state[1], m0=state[2])
    h_ref, C_ref, n_ref, m_ref = oracle.mlstm_stabilized(d["q"], d["k"], d["v"], d["i_tilde"],
                                                         d["f_tilde"], **kw)
    eh, eC, en = rel_err(host(h), h_ref), rel_err(host(C), C_ref), rel_err(host(n), n_ref)
    em = float(np.max(np.abs(host(m) - m_ref)))
    tol = TOL[d["dtype"]]
    say(f"[mlstm] {label}: err_h={eh:.3e} err_C={eC:.3e} err_n={en:.3e} |dm|={em:.2e} tol={tol:g}")
    assert eh <= tol and eC <= tol and en <= tol and em <= 1e-4 * max(1.0, np.abs(m_ref).max())


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,chunk", [(16, 16, 16), (64, 64, 64), (128, 32, 32), (32, 128, 64),
                                         (128, 128, 64), (64, 16, 16)])
def test_mlstm_shapes(path, dtype, dk, dv, chunk):
    d = mlstm_inputs(2, 2, 2 * chunk + 9, dk, dv, seed=dk + dv, dtype=dtype)
    _check(d, chunk, f"{dtype} dk={dk} dv={dv} C={chunk}", path=path)


@pytest.mark.parametrize("path", PATHS)
def test_mlstm_dk256_bf16(path):
    d = mlstm_inputs(1, 2, 150, 256, 256, seed=2, dtype="bf16")
    _check(d, 64, "bf16 dk=dv=256", path=path)


@pytest.mark.parametrize("dtype,chunk,B,dv", [("bf16", 32, 4, 256), ("bf16", 64, 4, 256), ("f32", 32, 8, 128)])
def test_mlstm_wide_batch(dtype, chunk, B, dv):
    """Enough (b, h) pairs that the workspace scan takes 32-column value tiles
    (B*H*d_v/32 = 256 workgroups)."""
    d = mlstm_inputs(B, 8, 2 * chunk + 5, 32, dv, seed=chunk + 7, dtype=dtype)
    _check(d, chunk, f"{dtype} wide batch B={B} H=8 dk=32 dv={dv} C={chunk}", path="ws")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T", [1, 7, 64, 65])
def test_mlstm_short_sequences(path, T):
    d = mlstm_inputs(1, 2, T, 64, 64, seed=T, dtype="bf16")
    _check(d, 64, f"bf16 T={T}", path=path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype,chunk", [("f32", 32), ("bf16", 32), ("bf16", 64)])
def test_mlstm_with_initial_state_and_large_gates(path, dtype, chunk):
    d = mlstm_inputs(2, 2, 100, 64, 64, seed=4, dtype=dtype)
    d["i_tilde"][:, :, 30] = 60.0          # one very strong write
    rng = np.random.default_rng(4)
    C0 = rng.standard_normal((2, 2, 64, 64)).astype(np.float32).astype(np.float64)
    n0 = np.abs(rng.standard_normal((2, 2, 64))).astype(np.float32).astype(np.float64)
    m0 = np.array([[0.5, -1.0], [2.0, 0.0]])
    _check(d, chunk, f"{dtype} C={chunk} with initial state, i_tilde = 60", state=(C0, n0, m0), path=path)


@pytest.mark.parametrize("path", PATHS)
def test_full_size_mlstm_sampled_heads(path):
    import torch
    c = CONFIGS["mlstm_8k"]
    d = mlstm_inputs(c["B"], c["H"], c["T"], c["dk"], c["dv"], seed=0, dtype=c["dtype"])
    h, C, n, m = _run(d, c["chunk"], path=path)
    torch.cuda.synchronize()
    h, C = host(h), host(C)
    for (bi, hi) in [(0, 0), (1, 7)]:
        sl = lambda x: x[bi:bi + 1, hi:hi + 1]
        h_ref, C_ref, _, _ = oracle.mlstm_stabilized(*(sl(d[x]) for x in ("q", "k", "v", "i_tilde", "f_tilde")))
        eh, eC = rel_err(sl(h), h_ref), rel_err(sl(C), C_ref)
        say(f"[mlstm] {path} full-size head (b={bi},h={hi}): err_h={eh:.3e} err_C={eC:.3e}")
        assert eh <= TOL["bf16"] and eC <= TOL["bf16"]


def test_mlstm_ws_agrees_with_fused_and_chains_state():
    """Two halves through gdr_mlstm_fwd_ws with the state handed over equal one
    call on the whole sequence (and the fused kernel) to within rounding."""
    import torch
    import matrix_memory_rnn_amd as gdr
    d = mlstm_inputs(2, 2, 200, 64, 64, seed=31, dtype="f32")
    t = lambda x, sl=slice(None): dev(d[x][:, :, sl], "f32")
    args = lambda sl: (t("q", sl), t("k", sl), t("v", sl), t("i_tilde", sl), t("f_tilde", sl))
    h_all, C_all, n_all, m_all = gdr.gdr_mlstm_fwd_ws(*args(slice(None)), chunk=32)
    h1, C1, n1, m1 = gdr.gdr_mlstm_fwd_ws(*args(slice(0, 96)), chunk=32)
    h2, C2, n2, m2 = gdr.gdr_mlstm_fwd_ws(*args(slice(96, None)), C1, n1, m1, chunk=32)
    hf, Cf, nf, mf = gdr.gdr_mlstm_fwd(*args(slice(None)), chunk=32)
    torch.cuda.synchronize()
    h_cat = np.concatenate([host(h1), host(h2)], axis=2)
    assert rel_err(h_cat, host(h_all)) < 1e-5 and rel_err(host(C2), host(C_all)) < 1e-5
    assert np.max(np.abs(host(m2) - host(m_all))) < 1e-4
    assert rel_err(host(h_all), host(hf)) < 1e-5 and rel_err(host(C_all), host(Cf)) < 1e-5


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("B,H,dv", [(1, 2, 64), (4, 8, 256)])
def test_mlstm_state_in_place(path, B, H, dv):
    """C_out may be C0 (each workgroup reads and writes only its own value
    columns); n_out and m_out are separate. The in-place call equals the one
    with separate outputs bit for bit. (4, 8, 256) takes 32-column tiles."""
    import torch
    import matrix_memory_rnn_amd as gdr
    d = mlstm_inputs(B, H, 100, 32, dv, seed=12, dtype="bf16")
    q, k, v = (dev(d[n], "bf16") for n in ("q", "k", "v"))
    it, ft = dev(d["i_tilde"]), dev(d["f_tilde"])
    rng = np.random.default_rng(12)
    C0 = dev(rng.standard_normal((B, H, 32, dv)))
    n0 = dev(np.abs(rng.standard_normal((B, H, 32))))
    m0 = dev(rng.uniform(-1, 2, (B, H)))
    fn = gdr.gdr_mlstm_fwd if path == "fused" else gdr.gdr_mlstm_fwd_ws
    h1, C1, n1, m1 = fn(q, k, v, it, ft, C0, n0, m0, chunk=64)
    Cin = C0.clone()
    n_out, m_out = torch.empty_like(n0), torch.empty_like(m0)
    h2, C2, n2, m2 = fn(q, k, v, it, ft, Cin, n0, m0, chunk=64, C_out=Cin, n_out=n_out, m_out=m_out)
    torch.cuda.synchronize()
    assert C2.data_ptr() == Cin.data_ptr()
    assert torch.equal(h1, h2) and torch.equal(C1, Cin) and torch.equal(n1, n_out) and torch.equal(m1, m_out)


@pytest.mark.parametrize("path", PATHS)
def test_mlstm_value_column_permutation(path):
    """Each value column of h and C depends only on the same column of v and
    C0 (the normaliser and stabiliser are shared by all columns): permuting
    the value columns of the inputs permutes the outputs' columns, exactly."""
    import torch
    import matrix_memory_rnn_amd as gdr
    B, H, T, dk, dv = 1, 2, 150, 64, 64
    d = mlstm_inputs(B, H, T, dk, dv, seed=14, dtype="bf16")
    rng = np.random.default_rng(14)
    C0 = rng.standard_normal((B, H, dk, dv))
    n0 = np.abs(rng.standard_normal((B, H, dk)))
    m0 = rng.uniform(-1, 2, (B, H))
    perm = rng.permutation(dv)
    fn = gdr.gdr_mlstm_fwd if path == "fused" else gdr.gdr_mlstm_fwd_ws
    args = lambda vv, cc: (dev(d["q"], "bf16"), dev(d["k"], "bf16"), dev(vv, "bf16"), dev(d["i_tilde"]),
                           dev(d["f_tilde"]), dev(cc), dev(n0), dev(m0))
    h1, C1, n1, m1 = fn(*args(d["v"], C0), chunk=64)
    h2, C2, n2, m2 = fn(*args(d["v"][..., perm], C0[..., perm]), chunk=64)
    torch.cuda.synchronize()
    p = torch.as_tensor(perm, device=h1.device)
    assert torch.equal(h2, h1.index_select(-1, p)) and torch.equal(C2, C1.index_select(-1, p))
    assert torch.equal(n2, n1) and torch.equal(m2, m1)


@pytest.mark.parametrize("dv", [64, 256])
def test_mlstm_bf16_split_at_chunk_boundary_chains_exactly(dv):
    """Two calls split at a chunk boundary, the state handed over, give the
    whole-sequence result bit for bit on the workspace path: the second call
    starts from the same fp32 state the first call's scan carried."""
    import torch
    import matrix_memory_rnn_amd as gdr
    d = mlstm_inputs(1, 4, 300, 64, dv, seed=21, dtype="bf16")
    t = lambda x, sl: dev(d[x][:, :, sl], "bf16")
    g = lambda x, sl: dev(d[x][:, :, sl])
    args = lambda sl: (t("q", sl), t("k", sl), t("v", sl), g("i_tilde", sl), g("f_tilde", sl))
    h, C, n, m = gdr.gdr_mlstm_fwd_ws(*args(slice(None)), chunk=64)
    h1, C1, n1, m1 = gdr.gdr_mlstm_fwd_ws(*args(slice(0, 128)), chunk=64)
    h2, C2, n2, m2 = gdr.gdr_mlstm_fwd_ws(*args(slice(128, None)), C1, n1, m1, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([h1, h2], dim=2), h)
    assert torch.equal(C2, C) and torch.equal(n2, n) and torch.equal(m2, m)
