"""Parity where the chunkwise method is numerically hard (HIP, gfx950, against
the float64 oracle).

* Ill-conditioned chunk systems. Trained models give unit lower-triangular
  chunk matrices T = I + L_strict with 2-norm condition numbers up to about
  40 ("Muir: ...", §5.2.4, numerical stability), while random unit keys in 128
  dimensions are nearly orthogonal and give about 2.3. Keys clustered around
  a few shared directions with erase gates near 2 reproduce (and exceed) the
  trained regime; the condition numbers are computed by the oracle and
  asserted before the GPU runs.
* The in-block factorisation at its limit: 16-row blocks whose total decay
  is 2^-48 or exactly the 2^-60 guard, which still take the factored path
  P_t * (Qs_s / G) with its largest ratios.
"""
import numpy as np
import pytest

import oracle
from oracle.gdn2 import chunk_condition_numbers
from synth import gdn2_inputs, gdn2_inputs_correlated
from tests.gpu_util import check_outputs, dev, host, rel_err, say

pytestmark = pytest.mark.gpu

PATHS = ["fused", "ws"]


def _fn(path):
    import matrix_memory_rnn_amd as gdr
    return gdr.gdr_chunk_fwd if path == "fused" else gdr.gdr_chunk_fwd_ws


def _chunk_parity(d, chunk, path, label, tol=None):
    import torch
    t = lambda x: dev(d[x], d["dtype"])
    S0 = dev(d["S0"]) if d["S0"] is not None else None
    o, S = _fn(path)(t("q"), t("k"), t("v"), t("alpha"), t("b"), t("w"), S0, chunk=chunk)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gdn2_recurrent(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], S0=d["S0"])
    return check_outputs(host(o), o_ref, host(S), S_ref, d["dtype"], label, tol)


def _kappa(d, chunk, lo):
    kap = chunk_condition_numbers(d["k"], d["alpha"], d["b"], chunk)
    say(f"[hard] chunk systems: kappa_2 median {np.median(kap):.1f} p90 {np.percentile(kap, 90):.1f} "
        f"max {kap.max():.1f} over {kap.size}")
    assert kap.max() >= lo
    return kap


# (n_dirs, b_mu, tol): 4 directions give kappa_2 of about 40-80 (the trained
# regime and a little beyond) and are held to the method's 2e-2; 2 directions
# give about 100-130, three times the largest value the pages report, where
# the two-kernel path's bf16 solve operands cost more (2.1e-2 measured on
# S_T) and the bar is 3e-2
CORR = {"kappa40": (4, 2.0, 2e-2), "kappa60": (4, 3.0, 2e-2), "kappa110": (2, 3.0, 3e-2)}


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", list(CORR))
def test_ill_conditioned_chunks_bf16(path, case):
    """d = 128, C = 64 (the 4K workload's head shape), bf16 inputs, fp32 state,
    a ragged tail and a nonzero initial state."""
    n_dirs, b_mu, tol = CORR[case]
    d = gdn2_inputs_correlated(2, 8, 1024 + 37, 128, 128, n_dirs=n_dirs, b_mu=b_mu, seed=17,
                               dtype="bf16", s0_std=0.02)
    _kappa(d, 64, 30.0)
    _chunk_parity(d, 64, path, f"[hard] {path} bf16 {case} B=2 H=8 T=1061 d=128 C=64", tol)


@pytest.mark.parametrize("path", PATHS)
def test_ill_conditioned_chunks_f32(path):
    d = gdn2_inputs_correlated(1, 4, 300, 64, 64, n_dirs=4, b_mu=3.0, seed=18, dtype="f32", s0_std=0.1)
    _kappa(d, 32, 30.0)
    _chunk_parity(d, 32, path, f"[hard] {path} f32 kappa60 B=1 H=4 T=300 d=64 C=32")


def test_ill_conditioned_wide_batch_fragment_order():
    """Enough heads that the two-kernel path takes its fragment-order record
    and 32x32x16 scan (B*H*d_v/32 >= 256 workgroups)."""
    d = gdn2_inputs_correlated(4, 16, 512 + 9, 128, 128, n_dirs=4, b_mu=3.0, seed=19, dtype="bf16",
                               s0_std=0.02)
    _kappa(d, 64, 30.0)
    _chunk_parity(d, 64, "ws", "[hard] ws bf16 kappa60 wide B=4 H=16 T=521 d=128 C=64")


def test_ill_conditioned_decode():
    """The decode step on the same kind of inputs (bf16), 200 steps from a
    nonzero state; every step's output and the final state are checked."""
    import torch
    import matrix_memory_rnn_amd as gdr
    d = gdn2_inputs_correlated(3, 4, 200, 128, 128, n_dirs=4, b_mu=3.0, seed=20, dtype="bf16", s0_std=0.05)
    S = dev(d["S0"])
    outs = []
    for t in range(200):
        x = [dev(np.ascontiguousarray(d[n][:, :, t]), "bf16") for n in ("q", "k", "v", "alpha", "b", "w")]
        outs.append(gdr.gdr_decode_step(*x, S))
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=2)
    o_ref, S_ref = oracle.gdn2_recurrent(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], S0=d["S0"])
    check_outputs(host(o), o_ref, host(S), S_ref, "bf16", "[hard] decode bf16 kappa60 N=3 H=4 200 steps")


def _guard_inputs(dtype, B, H, T, dk, dv, chunk, seed):
    d = gdn2_inputs(B, H, T, dk, dv, alpha_mu=3.5, alpha_sigma=1.2, seed=seed, dtype=dtype, s0_std=0.2)
    a = d["alpha"]
    # block 1 of chunk 0, channels 0-7: sixteen factors of 2^-3, block total 2^-48
    a[:, :, 16:32, 0:8] = 2.0 ** -3
    # block 0 of chunk 1, channels 8-11: fifteen factors of 2^-4 and one 1, total 2^-60 (the guard)
    a[:, :, chunk:chunk + 15, 8:12] = 2.0 ** -4
    a[:, :, chunk + 15, 8:12] = 1.0
    # the last block of chunk 1: one factor 2^-20 per channel 20-27 at its third row
    a[:, :, 2 * chunk - 14, 20:28] = 2.0 ** -20
    return d


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_guard_boundary_factored_path(path, dtype):
    """Blocks whose total decay is 2^-48 or exactly 2^-60 still take the
    factored in-block path, where Qs_s / G reaches 2^48..2^60."""
    chunk = 32 if (path == "fused" and dtype == "f32") else 64
    d = _guard_inputs(dtype, 1, 3, 3 * chunk + 11, 64, 64, chunk, 30)
    _chunk_parity(d, chunk, path, f"[hard] {path} {dtype} guard boundary C={chunk}")


def test_guard_boundary_wide_batch_fragment_order():
    d = _guard_inputs("bf16", 4, 16, 3 * 64 + 11, 128, 128, 64, 31)
    _chunk_parity(d, 64, "ws", "[hard] ws bf16 guard boundary wide B=4 H=16 d=128")


def test_fused_and_two_kernel_paths_agree_on_ill_conditioned_inputs():
    import torch
    d = gdn2_inputs_correlated(1, 4, 700, 128, 128, n_dirs=4, b_mu=3.0, seed=21, dtype="bf16", s0_std=0.02)
    t = lambda x: dev(d[x], "bf16")
    args = [t(x) for x in ("q", "k", "v", "alpha", "b", "w")] + [dev(d["S0"])]
    o1, S1 = _fn("fused")(*args, chunk=64)
    o2, S2 = _fn("ws")(*args, chunk=64)
    torch.cuda.synchronize()
    e = rel_err(host(o1), host(o2))
    say(f"[hard] fused vs ws on kappa60 inputs: {e:.3e}")
    assert e < 2e-2
