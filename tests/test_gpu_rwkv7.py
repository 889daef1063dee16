"""Parity of RWKV-7's generalized delta rule on the GPU (gdr_rwkv7_fwd, two
kernels through a workspace, and gdr_rwkv7_decode_step) with the float64
oracle ("Exponential gates and matrix memory: xLSTM and RWKV-7", §13.3), and
the page's eviction demo run through the GPU kernels."""
import numpy as np
import pytest

import oracle
from synth import rwkv7_inputs
from tests.gpu_util import check_outputs, dev, host, rel_err, say

pytestmark = pytest.mark.gpu

SEQ = ("q", "w", "a", "kw", "u")


def _run(d, chunk):
    import matrix_memory_rnn_amd as gdr
    x = {n: dev(d[n], d["dtype"]) for n in SEQ}
    S0 = None if d["S0"] is None else dev(d["S0"])
    return gdr.gdr_rwkv7_fwd(x["q"], x["w"], x["a"], dev(d["c"]), x["kw"], x["u"], S0, chunk=chunk)


def _ref(d):
    return oracle.rwkv7_recurrent(d["q"], d["w"], d["a"], d["c"], d["kw"], d["u"], S0=d["S0"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,chunk", [(16, 16, 16), (32, 64, 32), (64, 32, 16), (128, 128, 32), (64, 64, 32)])
def test_rwkv7_chunk_parity(dtype, dk, dv, chunk):
    import torch
    d = rwkv7_inputs(2, 2, 3 * chunk + 7, dk, dv, seed=dk + dv + chunk, dtype=dtype, s0_std=0.1)
    o, S = _run(d, chunk)
    torch.cuda.synchronize()
    o_ref, S_ref = _ref(d)
    check_outputs(host(o), o_ref, host(S), S_ref, dtype, f"[rwkv7] {dtype} dk={dk} dv={dv} C={chunk}")


def test_rwkv7_long_sequence_bf16():
    import torch
    d = rwkv7_inputs(1, 4, 1000, 128, 128, seed=3, dtype="bf16", s0_std=0.02)
    o, S = _run(d, 32)
    torch.cuda.synchronize()
    o_ref, S_ref = _ref(d)
    check_outputs(host(o), o_ref, host(S), S_ref, "bf16", "[rwkv7] bf16 B=1 H=4 T=1000 d=128 C=32")


def test_rwkv7_chunk_sizes_agree_and_split_state():
    import torch
    import matrix_memory_rnn_amd as gdr
    d = rwkv7_inputs(1, 2, 200, 64, 64, seed=4, dtype="f32", s0_std=0.1)
    o16, S16 = _run(d, 16)
    o32, S32 = _run(d, 32)
    x = {n: dev(d[n], "f32") for n in SEQ}
    c = dev(d["c"])
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    o1, S1 = gdr.gdr_rwkv7_fwd(*(sl(x[n], 0, 96) for n in ("q", "w", "a")), sl(c, 0, 96),
                               *(sl(x[n], 0, 96) for n in ("kw", "u")), dev(d["S0"]), chunk=32)
    o2, S2 = gdr.gdr_rwkv7_fwd(*(sl(x[n], 96, 200) for n in ("q", "w", "a")), sl(c, 96, 200),
                               *(sl(x[n], 96, 200) for n in ("kw", "u")), S1, chunk=32)
    torch.cuda.synchronize()
    assert rel_err(host(o16), host(o32)) < 1e-5 and rel_err(host(S16), host(S32)) < 1e-5
    assert rel_err(np.concatenate([host(o1), host(o2)], axis=2), host(o32)) < 1e-5
    assert rel_err(host(S2), host(S32)) < 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rwkv7_decode_steps_and_equal_to_chunk(dtype):
    import torch
    import matrix_memory_rnn_amd as gdr
    d = rwkv7_inputs(3, 2, 40, 128, 64, seed=5, dtype=dtype, s0_std=0.1)
    S = dev(d["S0"])
    outs = []
    for t in range(40):
        x = [dev(np.ascontiguousarray(d[n][:, :, t]), dtype) for n in ("q", "w", "a")]
        y = [dev(np.ascontiguousarray(d[n][:, :, t]), dtype) for n in ("kw", "u")]
        outs.append(gdr.gdr_rwkv7_decode_step(*x, dev(np.ascontiguousarray(d["c"][:, :, t])), *y, S))
    torch.cuda.synchronize()
    o = np.stack([host(x) for x in outs], axis=2)
    o_ref, S_ref = _ref(d)
    check_outputs(o, o_ref, host(S), S_ref, dtype, f"[rwkv7] decode {dtype} 40 steps")
    if dtype == "f32":
        o_c, S_c = _run(d, 16)
        torch.cuda.synchronize()
        assert rel_err(o, host(o_c)) < 1e-5 and rel_err(host(S), host(S_c)) < 1e-5


def test_rwkv7_eviction_demo_on_gpu():
    """The page's eviction demo (c = 0.1, T = 30) through the chunk kernels in
    fp32: with the removal aimed at k_A the retrieval k_A S_T shrinks to
    (1 - c)^T |v_A| = 0.028576 for |v_A| = 0.674096; locked to the write keys
    it stays at 0.674096."""
    import torch
    import matrix_memory_rnn_amd as gdr
    T, dk, dv, c = 30, 16, 16, 0.1
    rng = np.random.default_rng(3)
    kA = np.zeros(dk)
    kA[0] = 1.0
    vA = rng.standard_normal(dv)
    vA *= 0.674096 / np.linalg.norm(vA)
    keys = rng.standard_normal((T, dk))
    keys[:, 0] = 0.0
    keys /= np.linalg.norm(keys, axis=-1, keepdims=True)
    vals = rng.standard_normal((T, dv))
    S0 = dev(np.outer(kA, vA)[None, None])
    sh = lambda x: dev(x[None, None], "f32")
    res = []
    for direction in (np.tile(kA, (T, 1)), keys):
        _, S = gdr.gdr_rwkv7_fwd(sh(np.zeros((T, dk))), sh(np.ones((T, dk))), sh(direction),
                                 dev(np.full((1, 1, T), c)), sh(keys), sh(vals), S0, chunk=16)
        torch.cuda.synchronize()
        res.append(np.linalg.norm(kA @ host(S)[0, 0]))
    say(f"[rwkv7] eviction demo: aimed {res[0]:.6f} locked {res[1]:.6f}")
    assert abs(res[0] - 0.028576) < 1e-6 and abs(res[1] - 0.674096) < 1e-6


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rwkv7_strong_decay_block_takes_exact_factors(dtype):
    """Channels whose decay falls below 2^-60 within one 16-token block: the
    kernel's Gram matrices use exact pairwise decays for that block instead of
    the block-pivot factors (which would exceed fp32 range there)."""
    import torch
    d = rwkv7_inputs(1, 2, 80, 64, 32, seed=11, dtype=dtype, s0_std=0.1)
    w = d["w"].copy()
    w[:, :, 16:32, :8] = 0.01            # 0.01^16 = 1e-32 in one block of chunk 0
    w[:, 1, 40:56, 20:30] = 0.02         # and inside chunk 1 for head 1
    from synth import round_to
    d["w"] = round_to(w, dtype)
    for chunk in (16, 32):
        o, S = _run(d, chunk)
        torch.cuda.synchronize()
        o_ref, S_ref = _ref(d)
        check_outputs(host(o), o_ref, host(S), S_ref, dtype, f"[rwkv7] {dtype} strong decay C={chunk}")
