"""The entry points under HIP graph capture: the library enqueues only kernel
launches on the caller's stream (no allocation, no memset, no
synchronisation), so a captured call replays to the same results as the
eager one. Each graph is replayed several times with eager work and
synchronisation in between, and every replay is checked."""
import numpy as np
import pytest

from synth import gdn2_inputs, mlstm_inputs
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _capture(fn):
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("B,H", [(2, 4), (2, 64)])
def test_chunk_fwd_ws_graph_replays(B, H):
    import torch
    import matrix_memory_rnn_amd as gdr
    T, dk, dv, C = 150, 128, 128, 64
    d = gdn2_inputs(B, H, T, dk, dv, alpha_mu=4.0, alpha_sigma=1.5, seed=51, dtype="bf16", s0_std=0.1)
    x = [dev(d[n], "bf16") for n in ("q", "k", "v", "alpha", "b", "w")]
    S0 = dev(d["S0"])
    ws = torch.empty(gdr.gdr_chunk_workspace_size(B, H, T, dk, dv, C, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    o_e, S_e = gdr.gdr_chunk_fwd_ws(*x, S0, chunk=C, workspace=ws)
    o_g = torch.empty_like(o_e)
    S_g = torch.empty_like(S_e)
    g = _capture(lambda: gdr.gdr_chunk_fwd_ws(*x, S0, chunk=C, o=o_g, S_out=S_g, workspace=ws))
    for r in range(3):
        o_g.fill_(float("nan"))
        S_g.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()    # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"[graph] chunk ws B={B} H={H} replay {r}: equal={torch.equal(o_g, o_e) and torch.equal(S_g, S_e)}")
        assert torch.equal(o_g, o_e) and torch.equal(S_g, S_e)
        del junk


def test_decode_graph_replays_advance_the_state():
    """A captured decode step updates S in place on every replay: three
    replays equal three eager steps."""
    import torch
    import matrix_memory_rnn_amd as gdr
    N, H, dk, dv = 8, 4, 128, 128
    rng = np.random.default_rng(5)

    def unit(shape):
        z = rng.standard_normal(shape)
        s = z / (1 + np.exp(-z))
        return s / np.linalg.norm(s, axis=-1, keepdims=True)

    sig = lambda z: 1 / (1 + np.exp(-z))
    x = [dev(unit((N, H, dk)), "bf16"), dev(unit((N, H, dk)), "bf16"),
         dev(rng.standard_normal((N, H, dv)), "bf16"),
         dev(sig(4 + 1.5 * rng.standard_normal((N, H, dk))), "bf16"),
         dev(sig(rng.standard_normal((N, H, dk))), "bf16"), dev(sig(rng.standard_normal((N, H, dv))), "bf16")]
    S0 = dev(0.05 * rng.standard_normal((N, H, dk, dv)))
    S_e = S0.clone()
    outs = []
    for _ in range(3):
        outs.append(gdr.gdr_decode_step(*x, S_e).clone())
    S_g = S0.clone()
    o_g = torch.empty_like(outs[0])
    g = _capture(lambda: gdr.gdr_decode_step(*x, S_g, o=o_g))
    S_g.copy_(S0)            # the warm-up before the capture advanced it
    torch.cuda.synchronize()
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, outs[r])
    assert torch.equal(S_g, S_e)


def test_mlstm_fwd_ws_graph_replays():
    import torch
    import matrix_memory_rnn_amd as gdr
    B, H, T, dk, dv, C = 1, 4, 130, 256, 256, 64
    d = mlstm_inputs(B, H, T, dk, dv, seed=6, dtype="bf16")
    q, k, v = (dev(d[n], "bf16") for n in ("q", "k", "v"))
    it, ft = dev(d["i_tilde"]), dev(d["f_tilde"])
    ws = torch.empty(gdr.gdr_mlstm_workspace_size(B, H, T, dk, dv, C, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    h_e, C_e, n_e, m_e = gdr.gdr_mlstm_fwd_ws(q, k, v, it, ft, chunk=C, workspace=ws)
    h_g = torch.empty_like(h_e)
    g = _capture(lambda: gdr.gdr_mlstm_fwd_ws(q, k, v, it, ft, chunk=C, h=h_g, return_state=False,
                                               workspace=ws))
    for _ in range(3):
        h_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h_g, h_e)


def test_mlstm_fwd_ws_segmented_graph_replays():
    """The segmented wide mLSTM scan (two launches, segment maps and the first
    segment's end state in the workspace) under capture, with an initial state
    and the final (C, n, m): every replay equals the eager call."""
    import torch
    import matrix_memory_rnn_amd as gdr
    B, H, T, dk, dv, C = 1, 2, 64 * 40 + 13, 64, 128, 64
    d = mlstm_inputs(B, H, T, dk, dv, seed=7, dtype="bf16")
    q, k, v = (dev(d[n], "bf16") for n in ("q", "k", "v"))
    it, ft = dev(d["i_tilde"]), dev(d["f_tilde"])
    rng = np.random.default_rng(7)
    C0 = dev(rng.standard_normal((B, H, dk, dv)))
    n0 = dev(np.abs(rng.standard_normal((B, H, dk))))
    m0 = dev(rng.uniform(-1, 2, (B, H)))
    ws = torch.empty(gdr.gdr_mlstm_workspace_size(B, H, T, dk, dv, C, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    h_e, C_e, n_e, m_e = gdr.gdr_mlstm_fwd_ws(q, k, v, it, ft, C0, n0, m0, chunk=C, workspace=ws)
    h_g, C_g, n_g, m_g = torch.empty_like(h_e), torch.empty_like(C_e), torch.empty_like(n_e), torch.empty_like(m_e)
    g = _capture(lambda: gdr.gdr_mlstm_fwd_ws(q, k, v, it, ft, C0, n0, m0, chunk=C, h=h_g, C_out=C_g, n_out=n_g,
                                               m_out=m_g, workspace=ws))
    for r in range(3):
        for x in (h_g, C_g, n_g, m_g):
            x.fill_(float("nan"))
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"[graph] segmented mLSTM replay {r}")
        assert torch.equal(h_g, h_e) and torch.equal(C_g, C_e) and torch.equal(n_g, n_e) and torch.equal(m_g, m_e)
