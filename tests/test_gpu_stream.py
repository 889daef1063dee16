"""Calls on a side stream: the binding passes the given stream to the library
and allocates its outputs and workspace on it, so memory the kernels still
use is not handed to other work on the current stream."""
import numpy as np
import pytest

from synth import gdn2_inputs, mlstm_inputs
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


def test_side_stream_chunk_and_mlstm_with_internal_allocations():
    import torch
    import matrix_memory_rnn_amd as gdr
    d = gdn2_inputs(2, 4, 700, 128, 128, alpha_mu=4.0, alpha_sigma=1.5, seed=90, dtype="bf16", s0_std=0.05)
    x = [dev(d[n], "bf16") for n in ("q", "k", "v", "alpha", "b", "w")] + [dev(d["S0"])]
    m = mlstm_inputs(2, 2, 300, 64, 64, seed=91, dtype="bf16")
    mx = [dev(m[n], "bf16") for n in ("q", "k", "v")] + [dev(m[n], "f32") for n in ("i_tilde", "f_tilde")]
    o_ref, S_ref = gdr.gdr_chunk_fwd_ws(*x, chunk=64)
    h_ref, C_ref, _, _ = gdr.gdr_mlstm_fwd_ws(*mx, chunk=64)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    outs = []
    for _ in range(3):
        o, S = gdr.gdr_chunk_fwd_ws(*x, chunk=64, stream=side)          # workspace allocated inside
        h, C, _, _ = gdr.gdr_mlstm_fwd_ws(*mx, chunk=64, stream=side)
        outs.append((o, S, h, C))
        # the current stream allocates and overwrites memory meanwhile; a block
        # the side-stream kernels still use must not be among it
        junk = [torch.full((1 << 22,), float(i), device="cuda") for i in range(24)]
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for o, S, h, C in outs:
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
        assert torch.equal(h, h_ref) and torch.equal(C, C_ref)


def test_side_stream_decode():
    import torch
    import matrix_memory_rnn_amd as gdr
    from synth import decode_inputs
    dd = decode_inputs(8, 4, 128, 128, step=0, dtype="bf16")
    x = [dev(dd[n], "bf16") for n in ("q", "k", "v", "alpha", "b", "w")]
    S0 = np.random.default_rng(5).standard_normal((8, 4, 128, 128)).astype(np.float32)
    Sa, Sb = torch.from_numpy(S0).cuda(), torch.from_numpy(S0).cuda()
    oa = gdr.gdr_decode_step(*x, Sa)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    ob = gdr.gdr_decode_step(*x, Sb, stream=side)
    side.synchronize()
    assert torch.equal(oa, ob) and torch.equal(Sa, Sb)
