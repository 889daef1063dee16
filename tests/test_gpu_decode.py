"""Parity of gdr_decode_step (HIP, gfx950) with the float64 oracle, and the
decode == chunk invariant."""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, decode_inputs, gdn2_inputs
from tests.gpu_util import TOKEN_TOL, TOL, dev, host, rel_err, say, token_err

pytestmark = pytest.mark.gpu


def _step(S, d):
    import matrix_memory_rnn_amd as gdr
    t = lambda x: dev(d[x], d["dtype"])
    return gdr.gdr_decode_step(t("q"), t("k"), t("v"), t("alpha"), t("b"), t("w"), S)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16)])
def test_decode_steps(dtype, dk, dv):
    import torch
    N, H, steps = 3, 2, 6
    rng = np.random.default_rng(dk * dv)
    S0 = (0.3 * rng.standard_normal((N, H, dk, dv))).astype(np.float32).astype(np.float64)
    S = dev(S0)
    S_ref = S0
    for st in range(steps):
        d = decode_inputs(N, H, dk, dv, step=st, seed=1, dtype=dtype, alpha_mu=2.0, alpha_sigma=1.0)
        o = _step(S, d)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.gdn2_decode(S_ref, d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"])
        eo = rel_err(host(o), o_ref)
        assert eo <= TOL[dtype], (st, eo)
    es = rel_err(host(S), S_ref)
    say(f"[decode] {dtype} dk={dk} dv={dv}: err_S={es:.3e}")
    assert es <= TOL[dtype]


def test_decode_equals_chunk():
    """T decode steps reproduce the chunkwise forward over the same T tokens."""
    import torch
    import matrix_memory_rnn_amd as gdr
    d = gdn2_inputs(2, 2, 40, 64, 64, alpha_mu=3.0, alpha_sigma=1.0, seed=3, dtype="f32", s0_std=0.2)
    t = lambda x: dev(d[x], "f32")
    full = [t(x) for x in ("q", "k", "v", "alpha", "b", "w")]
    o_c, S_c = gdr.gdr_chunk_fwd(*full, dev(d["S0"]), chunk=16)
    S = dev(d["S0"])
    outs = []
    for i in range(40):
        outs.append(gdr.gdr_decode_step(*[x[:, :, i].contiguous() for x in full], S))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, dim=2)
    assert rel_err(host(o_d), host(o_c)) < 5e-5 and rel_err(host(S), host(S_c)) < 5e-5


def test_full_size_decode_sampled_heads():
    """256 sequences x 16 heads, d = 128: four consecutive steps from a nonzero
    state (N(0, 0.05)); the oracle follows 256 of the 4096 states, spread over
    every sequence group and head."""
    import torch
    c = CONFIGS["decode"]
    N, H, dk, dv = c["N"], c["H"], c["dk"], c["dv"]
    rng = np.random.default_rng(77)
    S0 = (0.05 * rng.standard_normal((N, H, dk, dv))).astype(np.float32)
    S = torch.from_numpy(S0).cuda()
    flat = np.arange(0, N * H, 16) + np.arange(N * H // 16) % 16   # one state per 16, every head
    ni, hi = flat // H, flat % H
    S_ref = S0[ni, hi][None].astype(np.float64)
    for st in range(4):
        d = decode_inputs(N, H, dk, dv, step=st, seed=0, dtype=c["dtype"])
        o = host(_step(S, d))
        torch.cuda.synchronize()
        sl = lambda x: x[ni, hi][None]
        o_ref, S_ref = oracle.gdn2_decode(S_ref, *(sl(d[x]) for x in ("q", "k", "v", "alpha", "b", "w")))
        eo, to = rel_err(sl(o), o_ref), token_err(sl(o)[:, :, None], o_ref[:, :, None])
        say(f"[decode] full-size step {st}: err_o={eo:.3e} tok_o={to:.3e}")
        assert eo <= TOL["bf16"] and to <= TOKEN_TOL["bf16"]
    es = rel_err(host(S)[ni, hi][None], S_ref)
    say(f"[decode] full-size 256 sampled states: err_S={es:.3e}")
    assert es <= TOL["bf16"]
