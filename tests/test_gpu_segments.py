"""The sequence-segmented chunk scan (HIP, gfx950) against the float64 oracle.

With few (b, h, value tile) workgroups and a long chunk chain, the two-kernel
forward cuts each head's chunks into segments: every segment's affine map
S_end = P_g S_start + Q_g ("Muir: ...", §4.2 eq.(10) composed over the
segment) is found side by side, the segment start states follow in order, and
the segments are then scanned side by side from them. The plan depends on the
shapes only; these shapes take it (bf16, d and C multiples of 32, at least 32
chunks, at most 128 workgroups in the plain scan)."""
import numpy as np
import pytest

import oracle
from synth import gdn2_inputs, gdn2_inputs_correlated
from tests.gpu_util import check_outputs, dev, host, rel_err, say

pytestmark = pytest.mark.gpu

SEQ = ("q", "k", "v", "alpha", "b", "w")


# The segment maps take two 32-column tiles per workgroup where d_v/32 and
# d_k/32 are both even (the first and third shapes), one tile otherwise.
@pytest.mark.parametrize("B,H,T,dk,dv,chunk", [(1, 2, 64 * 40 + 13, 128, 128, 64),   # 2 segments of 21
                                               (1, 2, 32 * 70, 64, 32, 32),          # 4 segments of 18
                                               (2, 3, 64 * 64 + 5, 128, 64, 64),     # 6 units: 4 segments
                                               (1, 1, 32 * 300 + 31, 32, 32, 32)])   # 18 segments
def test_segmented_scan_parity(B, H, T, dk, dv, chunk):
    import torch
    import matrix_memory_rnn_amd as gdr
    d = gdn2_inputs(B, H, T, dk, dv, alpha_mu=4.0, alpha_sigma=1.5, seed=T + dk, dtype="bf16", s0_std=0.05)
    x = [dev(d[n], "bf16") for n in SEQ]
    S0 = dev(d["S0"])
    o, S = gdr.gdr_chunk_fwd_ws(*x, S0, chunk=chunk)
    # the plain scan (the no-allocation entry point never segments)
    o2, S2 = torch.empty_like(o), torch.empty_like(S)
    gdr.gdr_chunk_fwd_noalloc(*x, S0, chunk=chunk, o=o2, S_out=S2)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gdn2_recurrent(*(d[n] for n in SEQ), S0=d["S0"])
    check_outputs(host(o), o_ref, host(S), S_ref, "bf16", f"[seg] B={B} H={H} T={T} dk={dk} dv={dv} C={chunk}")
    e1, e2 = rel_err(host(o), host(o2)), rel_err(host(S), host(S2))
    say(f"[seg] segmented vs plain scan: o {e1:.3e} S {e2:.3e}")
    assert e1 < 1e-2 and e2 < 1e-2


def test_segmented_scan_ill_conditioned():
    import torch
    import matrix_memory_rnn_amd as gdr
    d = gdn2_inputs_correlated(1, 4, 4096, 128, 128, n_dirs=4, b_mu=3.0, seed=23, dtype="bf16", s0_std=0.02)
    o, S = gdr.gdr_chunk_fwd_ws(*(dev(d[n], "bf16") for n in SEQ), dev(d["S0"]), chunk=64)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gdn2_recurrent(*(d[n] for n in SEQ), S0=d["S0"])
    check_outputs(host(o), o_ref, host(S), S_ref, "bf16", "[seg] kappa60 B=1 H=4 T=4096 d=128 C=64")


def test_segmented_phase_entry_points_equal_one_call():
    import torch
    import matrix_memory_rnn_amd as gdr
    B, H, T, dk, dv, C = 1, 2, 64 * 48, 128, 128, 64
    d = gdn2_inputs(B, H, T, dk, dv, alpha_mu=4.0, alpha_sigma=1.5, seed=24, dtype="bf16", s0_std=0.05)
    x = [dev(d[n], "bf16") for n in SEQ]
    S0 = dev(d["S0"])
    o1, S1 = gdr.gdr_chunk_fwd_ws(*x, S0, chunk=C)
    ws = gdr.gdr_chunk_intra(*x, chunk=C)
    o2, S2 = torch.empty_like(o1), torch.empty_like(S1)
    gdr.gdr_chunk_scan(ws, S0, o2, S2, B=B, H=H, T=T, dk=dk, dv=dv, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_segmented_in_place_state_and_no_state():
    """S_out = S0 in place, and S_out / S0 absent, on the segmented path."""
    import torch
    import matrix_memory_rnn_amd as gdr
    d = gdn2_inputs(1, 2, 64 * 40, 64, 64, alpha_mu=4.0, alpha_sigma=1.5, seed=25, dtype="bf16", s0_std=0.05)
    x = [dev(d[n], "bf16") for n in SEQ]
    o_a, S_a = gdr.gdr_chunk_fwd_ws(*x, dev(d["S0"]), chunk=64)
    Sp = dev(d["S0"])
    o_b, _ = gdr.gdr_chunk_fwd_ws(*x, Sp, chunk=64, S_out=Sp)
    o_c, S_c = gdr.gdr_chunk_fwd_ws(*x, None, chunk=64)
    o_d, _ = gdr.gdr_chunk_fwd_ws(*x, None, chunk=64, return_state=False)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(S_a, Sp) and torch.equal(o_c, o_d)
    o_ref, S_ref = oracle.gdn2_recurrent(*(d[n] for n in SEQ))
    check_outputs(host(o_c), o_ref, host(S_c), S_ref, "bf16", "[seg] no initial state")
