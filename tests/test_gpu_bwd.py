"""Gradients of the chunkwise forward (gdr_chunk_bwd, HIP, gfx950) against the
float64 gradient oracle (reverse-mode differentiation of eq.(1) of "Muir: ...",
§2.1, pinned by finite differences), for a loss J = <dO, O> + <dS_T, S_T>.

Every gradient (dq, dk, dv, dalpha, db, dw, dS0) is compared per head by
relative Frobenius error against the method's bars: 1e-4 for float32 inputs,
2e-2 for bfloat16 inputs (whose backward reads the forward's bf16 record: Y,
U, M, Q_pi, K~ rounded to 8 bits; measured about 4e-3)."""
import numpy as np
import pytest

import oracle
from synth import gdn2_inputs, gdn2_inputs_correlated
from tests.gpu_util import dev, host, rel_err, say

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "alpha", "b", "w")
GRADS = ("dq", "dk", "dv", "dalpha", "db", "dw", "dS0")
BWD_TOL = {"f32": 1e-4, "bf16": 2e-2}


def _grads(d, dO, dS, chunk, **kw):
    import torch
    import matrix_memory_rnn_amd as gdr
    x = [dev(d[n], d["dtype"]) for n in NAMES]
    S0 = None if d["S0"] is None else dev(d["S0"])
    g = gdr.gdr_chunk_bwd(*x, S0, dev(dO, d["dtype"]), None if dS is None else dev(dS), chunk=chunk, **kw)
    torch.cuda.synchronize()
    return {n: host(t) for n, t in g.items() if t is not None}


def _check(d, chunk, label, seed=0, with_dS=True, tol=None):
    rng = np.random.default_rng(seed)
    B, H, T, dk = d["q"].shape
    dv = d["v"].shape[-1]
    from synth import round_to
    dO = round_to(rng.standard_normal((B, H, T, dv)), d["dtype"])
    dS = round_to(rng.standard_normal((B, H, dk, dv)), "f32") if with_dS else None
    g = _grads(d, dO, dS, chunk)
    ref = oracle.gdn2_grad(*(d[n] for n in NAMES), d["S0"], dO, dS)
    tol = BWD_TOL[d["dtype"]] if tol is None else tol
    errs = {n: rel_err(g[n], ref[n]) for n in GRADS}
    say(f"[bwd] {label}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + f" tol={tol:g}")
    for n in GRADS:
        assert np.all(np.isfinite(g[n])), n
        assert errs[n] <= tol, (n, errs[n])
    return g


@pytest.mark.parametrize("dk,dv,chunk", [(16, 16, 16), (32, 64, 32), (64, 32, 16), (128, 128, 32), (64, 64, 64)])
def test_bwd_f32(dk, dv, chunk):
    d = gdn2_inputs(1, 2, 3 * chunk + 7, dk, dv, alpha_mu=3.0, alpha_sigma=1.0, seed=dk + dv + chunk,
                    dtype="f32", s0_std=0.3)
    _check(d, chunk, f"f32 dk={dk} dv={dv} C={chunk}")


@pytest.mark.parametrize("dk,dv,chunk", [(128, 128, 64), (64, 128, 32), (32, 32, 16)])
def test_bwd_bf16(dk, dv, chunk):
    d = gdn2_inputs(1, 2, 4 * chunk + 9, dk, dv, alpha_mu=4.0, alpha_sigma=1.5, seed=dk + chunk, dtype="bf16",
                    s0_std=0.05)
    _check(d, chunk, f"bf16 dk={dk} dv={dv} C={chunk}")


def test_bwd_without_initial_state_or_final_gradient():
    d = gdn2_inputs(2, 2, 100, 64, 64, alpha_mu=3.0, alpha_sigma=1.0, seed=5, dtype="f32")
    _check(d, 32, "f32 S0 = 0, dS_T = 0", with_dS=False)


def test_bwd_ill_conditioned_f32():
    d = gdn2_inputs_correlated(1, 2, 200, 64, 64, n_dirs=4, b_mu=3.0, seed=6, dtype="f32", s0_std=0.1)
    _check(d, 32, "f32 correlated keys")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_strong_decay_blocks(dtype):
    """Channels whose decay falls below 2^-60 inside one 16-token block (the
    forward's and the backward's Gram factors take exact pairwise decays
    there), below 2^-20 across two blocks (the backward's exact factors), and
    to e^-12.8 inside one block (the backward's block factors, with in-block
    ratios up to e^12.8)."""
    from synth import round_to
    d = gdn2_inputs(1, 2, 150, 64, 64, alpha_mu=4.0, alpha_sigma=1.5, seed=12, dtype=dtype, s0_std=0.1)
    a = d["alpha"].copy()
    a[:, :, 16:32, :8] = 0.01
    a[:, 1, 72:88, 20:30] = 0.02
    a[:, 0, 96:112, 30:40] = 0.45
    d["alpha"] = round_to(a, dtype)
    _check(d, 32, f"{dtype} strong decay blocks")


def test_bwd_records_ready_equals_recompute():
    """A workspace whose records the two-kernel forward wrote (records_ready)
    gives the same gradients bit for bit as recomputing them."""
    import torch
    import matrix_memory_rnn_amd as gdr
    d = gdn2_inputs(1, 3, 150, 128, 128, alpha_mu=4.0, alpha_sigma=1.5, seed=7, dtype="bf16", s0_std=0.05)
    x = [dev(d[n], "bf16") for n in NAMES]
    S0 = dev(d["S0"])
    dO = dev(np.random.default_rng(1).standard_normal((1, 3, 150, 128)), "bf16")
    need = gdr.gdr_chunk_bwd_workspace_size(1, 3, 150, 128, 128, 64, torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    g1 = gdr.gdr_chunk_bwd(*x, S0, dO, chunk=64, workspace=ws)
    gdr.gdr_chunk_intra(*x, chunk=64, workspace=ws)
    g2 = gdr.gdr_chunk_bwd(*x, S0, dO, chunk=64, workspace=ws, records_ready=True)
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.equal(g1[n], g2[n]), n


def test_bwd_tiny_f32_config():
    """The tiny float32 workload (B=1, H=2, T=64, d=16, C=16)."""
    from synth import CONFIGS
    c = CONFIGS["tiny_f32"]
    d = gdn2_inputs(c["B"], c["H"], c["T"], c["dk"], c["dv"], alpha_mu=c["alpha_mu"], alpha_sigma=c["alpha_sigma"],
                    seed=0, dtype="f32")
    _check(d, c["chunk"], "tiny f32 workload", with_dS=False)


def test_bwd_full_size_4k_sampled_heads():
    """The 4K workload (B=4, H=16, T=4096, d=128, C=64, bf16) through the
    backward; the oracle differentiates two of its heads."""
    import torch
    import matrix_memory_rnn_amd as gdr
    from synth import CONFIGS, round_to
    c = CONFIGS["chunk_4k"]
    d = gdn2_inputs(c["B"], c["H"], c["T"], c["dk"], c["dv"], alpha_mu=c["alpha_mu"], alpha_sigma=c["alpha_sigma"],
                    seed=0, dtype="bf16")
    dO = round_to(np.random.default_rng(9).standard_normal((c["B"], c["H"], c["T"], c["dv"])), "bf16")
    x = [dev(d[n], "bf16") for n in NAMES]
    g = gdr.gdr_chunk_bwd(*x, None, dev(dO, "bf16"), chunk=c["chunk"])
    torch.cuda.synchronize()
    g = {n: host(t) for n, t in g.items()}
    for (bi, hi) in [(0, 3), (3, 12)]:
        sl = lambda a: a[bi:bi + 1, hi:hi + 1]
        ref = oracle.gdn2_grad(*(sl(d[n]) for n in NAMES), None, sl(dO))
        errs = {n: rel_err(sl(g[n]), ref[n]) for n in GRADS}
        say(f"[bwd] 4K workload head ({bi},{hi}): " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
        assert all(e <= BWD_TOL["bf16"] for e in errs.values())
