"""Parity of the Muir gate-prologue entry points (HIP, gfx950) with the float64
oracle: gdr_muir_chunk_fwd_ws (gates formed from logits inside the intra-chunk
kernel's load stage) and gdr_muir_decode_step ("Muir: ...", §2.1, §4.1
eq.(8)-(9))."""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, muir_inputs
from tests.gpu_util import check_outputs, dev, host, rel_err, say

pytestmark = pytest.mark.gpu

SEQ = ("q", "k", "v", "z_f", "z_b", "z_w")


def _run_chunk(d, chunk):
    import matrix_memory_rnn_amd as gdr
    x = [dev(d[n], d["dtype"]) for n in SEQ]
    zq = None if d["z_q"] is None else dev(d["z_q"], d["dtype"])
    gs = None if d["gamma_stat"] is None else dev(d["gamma_stat"])
    S0 = None if d["S0"] is None else dev(d["S0"])
    return gdr.gdr_muir_chunk_fwd_ws(*x, dev(d["a_log"]), zq, gs, S0, chunk=chunk)


def _ref(d):
    return oracle.muir_recurrent(*(d[n] for n in SEQ), d["a_log"], d["z_q"], d["gamma_stat"], S0=d["S0"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,chunk", [(16, 16, 16), (64, 64, 32), (128, 128, 64), (64, 128, 64), (32, 16, 16)])
def test_muir_chunk_shapes(dtype, dk, dv, chunk):
    import torch
    d = muir_inputs(2, 3, 3 * chunk + 5, dk, dv, seed=dk + dv + chunk, dtype=dtype, s0_std=0.1)
    o, S = _run_chunk(d, chunk)
    torch.cuda.synchronize()
    o_ref, S_ref = _ref(d)
    check_outputs(host(o), o_ref, host(S), S_ref, dtype, f"[muir] {dtype} dk={dk} dv={dv} C={chunk}")


@pytest.mark.parametrize("with_zq,with_gamma", [(False, False), (False, True), (True, False)])
def test_muir_optional_gain_inputs(with_zq, with_gamma):
    import torch
    d = muir_inputs(1, 4, 150, 64, 64, seed=5, dtype="bf16", with_zq=with_zq, with_gamma=with_gamma, s0_std=0.1)
    o, S = _run_chunk(d, 64)
    torch.cuda.synchronize()
    o_ref, S_ref = _ref(d)
    check_outputs(host(o), o_ref, host(S), S_ref, "bf16", f"[muir] z_q={with_zq} gamma_stat={with_gamma}")


def test_muir_wide_batch_fragment_order_and_strong_decay():
    """Enough heads for the fragment-order record; logits that push some decays
    to 1e-8 (a_log large) and some to 1 (z_f very negative)."""
    import torch
    d = muir_inputs(4, 16, 2 * 64 + 9, 128, 128, seed=6, dtype="bf16", s0_std=0.05)
    d["a_log"][3] = 3.0                        # rate e^3: alpha down to ~1e-9 at z_f ~ 1
    d["z_f"][:, 5, 40:60] = -60.0              # alpha = 1 to float precision
    o, S = _run_chunk(d, 64)
    torch.cuda.synchronize()
    o_ref, S_ref = _ref(d)
    check_outputs(host(o), o_ref, host(S), S_ref, "bf16", "[muir] wide B=4 H=16 d=128, strong and no decay")


def test_muir_chunk_equals_gdn2_on_the_same_gates_f32():
    """fp32: the prologue kernel and gdr_chunk_fwd_ws fed with the oracle's gates
    (rounded to fp32) and gamma * q agree to fp32 rounding."""
    import torch
    import matrix_memory_rnn_amd as gdr
    d = muir_inputs(2, 2, 200, 64, 32, seed=7, dtype="f32", s0_std=0.1)
    o1, S1 = _run_chunk(d, 32)
    a, b, w, g = oracle.muir_gates(d["z_f"], d["z_b"], d["z_w"], d["a_log"], d["z_q"], d["gamma_stat"])
    x = [dev(g * d["q"]), dev(d["k"]), dev(d["v"]), dev(a), dev(b), dev(w)]
    o2, S2 = gdr.gdr_chunk_fwd_ws(*x, dev(d["S0"]), chunk=32)
    torch.cuda.synchronize()
    eo, es = rel_err(host(o1), host(o2)), rel_err(host(S1), host(S2))
    say(f"[muir] prologue vs precomputed gates (f32): {eo:.3e} {es:.3e}")
    assert eo < 1e-5 and es < 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_muir_decode_steps(dtype):
    import torch
    import matrix_memory_rnn_amd as gdr
    d = muir_inputs(3, 4, 8, 128, 64, seed=8, dtype=dtype, s0_std=0.2)
    S = dev(d["S0"])
    S_ref = d["S0"]
    gs, al = dev(d["gamma_stat"]), dev(d["a_log"])
    outs, refs = [], []
    for t in range(8):
        sl = lambda n: np.ascontiguousarray(d[n][:, :, t])
        x = [dev(sl(n), dtype) for n in SEQ]
        outs.append(gdr.gdr_muir_decode_step(*x, al, S, dev(sl("z_q"), dtype), gs))
        o_ref, S_ref = oracle.muir_decode(S_ref, *(sl(n) for n in SEQ), d["a_log"], sl("z_q"), d["gamma_stat"])
        refs.append(o_ref)
    torch.cuda.synchronize()
    o = np.stack([host(x) for x in outs], axis=2)
    check_outputs(o, np.stack(refs, axis=2), host(S), S_ref, dtype, f"[muir] decode {dtype} 8 steps")


def test_muir_decode_equals_chunk():
    import torch
    import matrix_memory_rnn_amd as gdr
    d = muir_inputs(2, 2, 40, 64, 64, seed=9, dtype="f32", s0_std=0.2)
    o_c, S_c = _run_chunk(d, 16)
    S = dev(d["S0"])
    al, gs = dev(d["a_log"]), dev(d["gamma_stat"])
    outs = []
    for t in range(40):
        x = [dev(np.ascontiguousarray(d[n][:, :, t])) for n in SEQ]
        outs.append(gdr.gdr_muir_decode_step(*x, al, S, dev(np.ascontiguousarray(d["z_q"][:, :, t])), gs))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, dim=2)
    assert rel_err(host(o_d), host(o_c)) < 5e-5 and rel_err(host(S), host(S_c)) < 5e-5


def test_muir_full_size_4k_sampled_heads():
    """The 4K workload's shape (B=4, H=16, T=4096, d=128, C=64, bf16) with all
    seven logit/input streams; the oracle follows 8 heads."""
    import torch
    c = CONFIGS["chunk_4k"]
    d = muir_inputs(c["B"], c["H"], c["T"], c["dk"], c["dv"], seed=0, dtype="bf16")
    o, S = _run_chunk(d, 64)
    torch.cuda.synchronize()
    o, S = host(o), host(S)
    sel = [(0, 0), (0, 9), (1, 3), (1, 15), (2, 6), (2, 12), (3, 1), (3, 14)]
    bi, hi = np.array([x[0] for x in sel]), np.array([x[1] for x in sel])
    sl = lambda x: x[bi, hi][None]
    # per-head parameters follow the heads
    a_log, gs = d["a_log"][hi], d["gamma_stat"][hi]
    o_ref, S_ref = oracle.muir_recurrent(*(sl(d[n]) for n in SEQ), a_log, sl(d["z_q"]), gs)
    check_outputs(sl(o), o_ref, sl(S), S_ref, "bf16", "[muir] 4K workload, 8 heads")
