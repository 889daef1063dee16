"""gdr_chunk_fwd_noalloc (the chunk forward through the library's static
scratch array, no allocation) against gdr_chunk_fwd_ws (same kernels through a
caller workspace) and the float64 oracle: two calls in a row, the second on a
smaller input, so the second reuses scratch the first left behind."""
import numpy as np
import pytest

import oracle
from synth import gdn2_inputs
from tests.gpu_util import check_outputs, dev, host, say

pytestmark = pytest.mark.gpu


def _pair(B, H, T, dk, dv, chunk, dtype, seed):
    import torch
    import matrix_memory_rnn_amd as gdr
    d = gdn2_inputs(B, H, T, dk, dv, alpha_mu=4.0, alpha_sigma=1.5, seed=seed, dtype=dtype, s0_std=0.05)
    x = [dev(d[n], dtype) for n in ("q", "k", "v", "alpha", "b", "w")] + [dev(d["S0"])]
    o_ws, S_ws = gdr.gdr_chunk_fwd_ws(*x, chunk=chunk)
    torch.cuda.synchronize()
    o = torch.empty_like(o_ws)
    S = torch.empty_like(S_ws)
    before = torch.cuda.memory_allocated()
    gdr.gdr_chunk_fwd_noalloc(*x, chunk=chunk, o=o, S_out=S)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return d, o, S, o_ws, S_ws


@pytest.mark.parametrize("second", ["fragment_order", "row_major_f32"])
def test_noalloc_two_calls_second_smaller(second):
    import torch
    # first call: 64 heads of 1,000 tokens (d = 128, C = 64): 16 chunks x 74,240 B
    # per head, so the 64 MiB array takes 56 heads per group and the call runs
    # two groups
    d, o, S, o_ws, S_ws = _pair(4, 16, 1000, 128, 128, 64, "bf16", 70)
    say(f"[noalloc] first call B=4 H=16 T=1000: equal to ws: {torch.equal(o, o_ws) and torch.equal(S, S_ws)}")
    assert torch.equal(o, o_ws) and torch.equal(S, S_ws)
    sel = [(0, 0), (1, 7), (3, 15), (2, 9)]
    bi, hi = np.array([x[0] for x in sel]), np.array([x[1] for x in sel])
    sl = lambda x: x[bi, hi][None]
    o_ref, S_ref = oracle.gdn2_recurrent(*(sl(d[n]) for n in ("q", "k", "v", "alpha", "b", "w")), S0=sl(d["S0"]))
    check_outputs(sl(host(o)), o_ref, sl(host(S)), S_ref, "bf16", "[noalloc] first call, 4 heads vs oracle")
    # second call, smaller
    if second == "fragment_order":
        d2, o2, S2, o2_ws, S2_ws = _pair(1, 3, 130, 64, 64, 32, "bf16", 71)
        assert torch.equal(o2, o2_ws) and torch.equal(S2, S2_ws)
    else:
        d2, o2, S2, o2_ws, S2_ws = _pair(1, 2, 77, 32, 16, 16, "f32", 72)
    o2_ref, S2_ref = oracle.gdn2_recurrent(*(d2[n] for n in ("q", "k", "v", "alpha", "b", "w")), S0=d2["S0"])
    check_outputs(host(o2), o2_ref, host(S2), S2_ref, d2["dtype"], f"[noalloc] second call ({second})")
    check_outputs(host(o2), host(o2_ws), host(S2), host(S2_ws), d2["dtype"],
                  f"[noalloc] second call ({second}) vs gdr_chunk_fwd_ws")
