"""Parity of the chunkwise entry points (HIP, gfx950) with the float64 oracle:
gdr_chunk_fwd (one fused kernel) and gdr_chunk_fwd_ws (intra-chunk kernel over
all chunks, then the chunk scan, through a workspace).

Tolerances (max over heads of the relative Frobenius error of O and S_T):
1e-4 for float32 inputs, 2e-2 for bfloat16 inputs with float32 state; every
output row (token) is also bounded on its own, and float32 results element
by element (``tests/gpu_util.py``).
"""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, gdn2_inputs
from tests.gpu_util import TOL, check_outputs, dev, host, rel_err, say

pytestmark = pytest.mark.gpu


PATHS = ["fused", "ws"]


def _fn(path):
    import matrix_memory_rnn_amd as gdr
    return gdr.gdr_chunk_fwd if path == "fused" else gdr.gdr_chunk_fwd_ws


def _run(d, chunk, S0=None, S_out=None, path="ws"):
    t = lambda x: dev(d[x], d["dtype"])
    S0d = dev(S0 if S0 is not None else d["S0"], "f32") if (S0 is not None or d["S0"] is not None) else None
    o, S = _fn(path)(t("q"), t("k"), t("v"), t("alpha"), t("b"), t("w"), S0d, chunk=chunk, S_out=S_out)
    return o, S


def _check(d, chunk, label, tol=None, path="ws"):
    import torch
    label = f"[chunk] {path} {label}"
    o, S = _run(d, chunk, path=path)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gdn2_recurrent(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], S0=d["S0"])
    eo, es, _ = check_outputs(host(o), o_ref, host(S), S_ref, d["dtype"], label, tol)
    return eo, es


@pytest.mark.parametrize("path", PATHS)
def test_tiny_f32_config(path):
    c = CONFIGS["tiny_f32"]
    d = gdn2_inputs(c["B"], c["H"], c["T"], c["dk"], c["dv"], alpha_mu=c["alpha_mu"],
                    alpha_sigma=c["alpha_sigma"], seed=0, dtype="f32")
    _check(d, c["chunk"], "tiny_f32 B=1 H=2 T=64 d=16 C=16", path=path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,chunk", [(16, 16, 16), (32, 32, 32), (64, 64, 64), (128, 128, 32),
                                         (64, 128, 64), (128, 32, 16), (32, 16, 64), (128, 128, 64)])
def test_shapes_and_ragged_tail(path, dtype, dk, dv, chunk):
    if path == "fused" and dtype == "f32" and dk >= 64:
        chunk = min(chunk, 32)          # the fused kernel's fp32 operands need twice the LDS
    d = gdn2_inputs(2, 2, 3 * chunk + 7, dk, dv, alpha_mu=3.0, alpha_sigma=1.0, seed=dk + dv + chunk,
                    dtype=dtype, s0_std=0.3)
    _check(d, chunk, f"{dtype} dk={dk} dv={dv} C={chunk} T={3 * chunk + 7}", path=path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T", [1, 5, 16, 63, 65])
def test_short_sequences(path, T):
    d = gdn2_inputs(1, 3, T, 128, 128, alpha_mu=4.0, alpha_sigma=1.5, seed=T, dtype="bf16", s0_std=0.1)
    _check(d, 64, f"bf16 T={T}", path=path)


@pytest.mark.parametrize("path", PATHS)
def test_chunk_size_invariance(path):
    import torch
    d = gdn2_inputs(1, 2, 256, 32, 64, alpha_mu=3.0, alpha_sigma=1.0, seed=5, dtype="f32", s0_std=0.2)
    outs = [(host(o), host(S)) for o, S in (_run(d, C, path=path) for C in (16, 32, 64))]
    torch.cuda.synchronize()
    for o, S in outs[1:]:
        assert rel_err(o, outs[0][0]) < 5e-5 and rel_err(S, outs[0][1]) < 5e-5


@pytest.mark.parametrize("path", PATHS)
def test_split_sequence_state_passing(path):
    import torch
    d = gdn2_inputs(2, 2, 320, 128, 128, alpha_mu=4.0, alpha_sigma=1.5, seed=6, dtype="bf16", s0_std=0.05)
    o_full, S_full = _run(d, 64, path=path)
    first = {k: (v[:, :, :192] if isinstance(v, np.ndarray) and v.ndim == 4 else v) for k, v in d.items()}
    second = {k: (v[:, :, 192:] if isinstance(v, np.ndarray) and v.ndim == 4 else v) for k, v in d.items()}
    o1, S1 = _run(first, 64, path=path)
    t = lambda x: dev(second[x], "bf16")
    o2, S2 = _fn(path)(t("q"), t("k"), t("v"), t("alpha"), t("b"), t("w"), S1, chunk=64)
    torch.cuda.synchronize()
    o_cat = np.concatenate([host(o1), host(o2)], axis=2)
    assert rel_err(o_cat, host(o_full)) < 1e-2 and rel_err(host(S2), host(S_full)) < 1e-2
    # split at a chunk boundary: the second call starts from the fp32 state
    # the first one carried, so the results are the same bits
    assert torch.equal(torch.cat([o1, o2], dim=2), o_full) and torch.equal(S2, S_full)


@pytest.mark.parametrize("path", PATHS)
def test_in_place_state_and_determinism(path):
    import torch
    d = gdn2_inputs(2, 4, 200, 128, 128, alpha_mu=4.0, alpha_sigma=1.5, seed=7, dtype="bf16", s0_std=0.1)
    t = lambda x: dev(d[x], "bf16")
    args = [t(x) for x in ("q", "k", "v", "alpha", "b", "w")]
    f = _fn(path)
    S_a = dev(d["S0"])
    o_a, _ = f(*args, S_a, chunk=64, S_out=S_a)      # in place
    o_b, S_b = f(*args, dev(d["S0"]), chunk=64)
    o_c, S_c = f(*args, dev(d["S0"]), chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o_b, o_c) and torch.equal(S_b, S_c)            # bit-identical reruns
    assert torch.equal(o_a, o_b) and torch.equal(S_a, S_b)


@pytest.mark.parametrize("path", PATHS)
def test_linear_in_initial_state(path):
    """Eq.(10) of the Muir page: O and S_C are affine in S0. With v = 0 they are linear."""
    import torch
    d = gdn2_inputs(1, 2, 130, 32, 32, alpha_mu=3.0, alpha_sigma=1.0, seed=8, dtype="f32", s0_std=1.0)
    d["v"] = np.zeros_like(d["v"])
    rng = np.random.default_rng(0)
    S1 = rng.standard_normal(d["S0"].shape).astype(np.float32).astype(np.float64)
    S2 = rng.standard_normal(d["S0"].shape).astype(np.float32).astype(np.float64)
    o1, s1 = _run(d, 32, S0=S1, path=path)
    o2, s2 = _run(d, 32, S0=S2, path=path)
    o3, s3 = _run(d, 32, S0=(S1 + 2 * S2).astype(np.float32).astype(np.float64), path=path)
    torch.cuda.synchronize()
    assert rel_err(host(o3), host(o1) + 2 * host(o2)) < 1e-4
    assert rel_err(host(s3), host(s1) + 2 * host(s2)) < 1e-4


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("B,H", [(2, 4), (2, 64)])
def test_value_column_permutation(path, B, H):
    """Each value column of O and S_T depends only on the same column of v,
    w and S0 (eq.(1) of the Muir page acts on S from the left): permuting the
    value columns of the inputs permutes the outputs' columns. Across value
    tiles and workgroups the arithmetic of a column is the same, so the match
    is exact. (B, H) = (2, 64) takes the fragment-order scan."""
    import torch
    d = gdn2_inputs(B, H, 150, 128, 128, alpha_mu=4.0, alpha_sigma=1.5, seed=41, dtype="bf16", s0_std=0.1)
    perm = np.random.default_rng(3).permutation(128)
    o1, s1 = _run(d, 64, path=path)
    dp = dict(d)
    dp["v"], dp["w"], dp["S0"] = d["v"][..., perm], d["w"][..., perm], d["S0"][..., perm]
    o2, s2 = _run(dp, 64, path=path)
    torch.cuda.synchronize()
    p = torch.as_tensor(perm, device=o1.device)
    assert torch.equal(o2, o1.index_select(-1, p)) and torch.equal(s2, s1.index_select(-1, p))


@pytest.mark.parametrize("path", PATHS)
def test_alpha_exactly_one_and_zero_erase(path):
    d = gdn2_inputs(1, 2, 100, 64, 64, alpha_mu=30.0, alpha_sigma=0.1, seed=9, dtype="bf16", s0_std=0.1)
    assert np.all(d["alpha"] == 1.0)
    _check(d, 64, "bf16 alpha == 1", path=path)
    d["b"] = np.zeros_like(d["b"])
    _check(d, 64, "bf16 alpha == 1, b == 0 (linear attention)", path=path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiny_decay_takes_exact_in_block_path(path, dtype):
    """Some channels decay below 2^-60 within 16 tokens: the in-block factorisation
    would leave fp32 range, so those diagonal tiles take the exact product path."""
    d = gdn2_inputs(1, 2, 96, 64, 64, alpha_mu=3.0, alpha_sigma=1.0, seed=10, dtype=dtype, s0_std=0.2)
    d["alpha"][:, :, 20:40, :8] = 1e-4
    d["alpha"][:, 1, 50:52, 10:20] = 1e-30
    _check(d, 32, f"{dtype} tiny alpha", path=path)


def _head_parity(name, heads, path):
    """Full-size workload through one entry point; the oracle follows the
    listed (b, h) pairs (all of them at once, vectorised over heads)."""
    import torch
    c = CONFIGS[name]
    d = gdn2_inputs(c["B"], c["H"], c["T"], c["dk"], c["dv"], alpha_mu=c["alpha_mu"],
                    alpha_sigma=c["alpha_sigma"], seed=0, dtype=c["dtype"], s0_std=c["s0_std"])
    say(f"[chunk] {name}: inputs ready")
    o, S = _run(d, c["chunk"], path=path)
    torch.cuda.synchronize()
    o, S = host(o), host(S)
    bi = np.array([x[0] for x in heads])
    hi = np.array([x[1] for x in heads])
    sl = lambda x: x[bi, hi][None]
    o_ref, S_ref = oracle.gdn2_recurrent(*(sl(d[x]) for x in ("q", "k", "v", "alpha", "b", "w")),
                                         S0=None if d["S0"] is None else sl(d["S0"]))
    say(f"[chunk] {name}: oracle done over {len(heads)} heads")
    check_outputs(sl(o), o_ref, sl(S), S_ref, c["dtype"], f"[chunk] {path} {name} {len(heads)} heads")


@pytest.mark.parametrize("path", PATHS)
def test_full_size_chunk_4k_all_heads(path):
    c = CONFIGS["chunk_4k"]
    _head_parity("chunk_4k", [(b, h) for b in range(c["B"]) for h in range(c["H"])], path)


@pytest.mark.parametrize("path", PATHS)
def test_full_size_chunk_32k_sampled_heads(path):
    _head_parity("chunk_32k", [(0, 0), (0, 5), (0, 11), (0, 15)], path)


def test_workspace_reuse_and_agreement_with_fused_kernel():
    """One oversized workspace serves calls of different sizes in a row; the
    two-kernel and fused forms agree to within their rounding."""
    import torch
    import matrix_memory_rnn_amd as gdr
    need = gdr.gdr_chunk_workspace_size(2, 3, 333, 128, 128, 64, torch.bfloat16)
    ws = torch.empty(need + 4096, dtype=torch.uint8, device="cuda")
    for T, seed in ((333, 11), (70, 12)):
        d = gdn2_inputs(2, 3, T, 128, 128, alpha_mu=4.0, alpha_sigma=1.5, seed=seed, dtype="bf16", s0_std=0.1)
        t = lambda x: dev(d[x], "bf16")
        args = [t(x) for x in ("q", "k", "v", "alpha", "b", "w")] + [dev(d["S0"])]
        o_w, S_w = gdr.gdr_chunk_fwd_ws(*args, chunk=64, workspace=ws)
        o_f, S_f = gdr.gdr_chunk_fwd(*args, chunk=64)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.gdn2_recurrent(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], S0=d["S0"])
        say(f"[chunk] reuse T={T}: err_o={rel_err(host(o_w), o_ref):.3e} "
            f"ws-vs-fused={rel_err(host(o_w), host(o_f)):.3e}")
        assert rel_err(host(o_w), o_ref) <= TOL["bf16"] and rel_err(host(S_w), S_ref) <= TOL["bf16"]
        assert rel_err(host(o_w), host(o_f)) < 1e-2 and rel_err(host(S_w), host(S_f)) < 1e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_phase_entry_points_equal_one_call(dtype):
    """gdr_chunk_intra then gdr_chunk_scan give bit-identical results to
    gdr_chunk_fwd_ws (same kernels, same order)."""
    import torch
    import matrix_memory_rnn_amd as gdr
    B, H, T, dk, dv, C = 2, 3, 200, 128, 64, 64
    d = gdn2_inputs(B, H, T, dk, dv, alpha_mu=4.0, alpha_sigma=1.5, seed=21, dtype=dtype, s0_std=0.1)
    t = lambda x: dev(d[x], dtype)
    x = [t(n) for n in ("q", "k", "v", "alpha", "b", "w")]
    S0 = dev(d["S0"])
    o1, S1 = gdr.gdr_chunk_fwd_ws(*x, S0, chunk=C)
    ws = gdr.gdr_chunk_intra(*x, chunk=C)
    o2 = torch.empty_like(o1)
    S2 = torch.empty_like(S1)
    gdr.gdr_chunk_scan(ws, S0, o2, S2, B=B, H=H, T=T, dk=dk, dv=dv, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


# With bfloat16 inputs and d_k, d_v and C multiples of 32 the record is written
# in the fragment-major order read by the 32x32x16 scan (also for the narrow
# batches of the other tests); these shapes fill the GPU with its
# (b, h, 32 value columns) workgroups (B*H*d_v/32 >= 256).
@pytest.mark.parametrize("dk,dv,chunk", [(128, 128, 64), (64, 64, 32), (32, 32, 64), (128, 64, 64),
                                         (64, 128, 32)])
def test_wide_batch_fragment_order_path(dk, dv, chunk):
    heads = -(-256 // (dv // 32))
    B, H = 2, heads // 2
    T = 2 * chunk + 9
    d = gdn2_inputs(B, H, T, dk, dv, alpha_mu=3.5, alpha_sigma=1.2, seed=dk + 3 * dv + chunk,
                    dtype="bf16", s0_std=0.2)
    _check(d, chunk, f"bf16 wide B={B} H={H} dk={dk} dv={dv} C={chunk} T={T}", path="ws")


@pytest.mark.parametrize("dk,dv,chunk", [(64, 64, 16), (16, 64, 32)])
def test_wide_batch_staged_path(dk, dv, chunk):
    """Wide batches whose d_k or C is not a multiple of 32 take the staged scan
    with 32-column value tiles (the path also taken when a head's records pass
    2 GiB)."""
    heads = -(-256 // (dv // 32))
    B, H = 2, heads // 2
    T = 2 * chunk + 9
    d = gdn2_inputs(B, H, T, dk, dv, alpha_mu=3.5, alpha_sigma=1.2, seed=11 + dk + chunk,
                    dtype="bf16", s0_std=0.2)
    _check(d, chunk, f"bf16 wide staged B={B} H={H} dk={dk} dv={dv} C={chunk} T={T}", path="ws")


@pytest.mark.parametrize("dk,dv,chunk", [(128, 128, 64), (64, 64, 32)])
def test_wide_batch_tiny_decay_exact_path(dk, dv, chunk):
    """The fragment-order path with blocks whose decay leaves the in-block
    factorisation's range (exact products for those diagonal tiles)."""
    heads = -(-256 // (dv // 32))
    B, H = 2, heads // 2
    T = 3 * chunk + 5
    d = gdn2_inputs(B, H, T, dk, dv, alpha_mu=3.5, alpha_sigma=1.2, seed=7 + dk + chunk,
                    dtype="bf16", s0_std=0.2)
    # powers of two: exact in bf16, so the oracle sees the kernel's inputs
    d["alpha"][0, 1, 20:40, :8] = 2.0 ** -13
    d["alpha"][1, 3, chunk + 2:chunk + 4, 10:20] = 2.0 ** -100
    d["alpha"][1, H - 1, T - 7:T - 5, 3] = 0.0
    _check(d, chunk, f"bf16 wide tiny alpha B={B} H={H} dk={dk} dv={dv} C={chunk} T={T}", path="ws")


def test_wide_batch_phase_entry_points_equal_one_call():
    import torch
    import matrix_memory_rnn_amd as gdr
    B, H, T, dk, dv, C = 4, 16, 150, 128, 128, 64
    d = gdn2_inputs(B, H, T, dk, dv, alpha_mu=4.0, alpha_sigma=1.5, seed=22, dtype="bf16", s0_std=0.1)
    x = [dev(d[n], "bf16") for n in ("q", "k", "v", "alpha", "b", "w")]
    S0 = dev(d["S0"])
    o1, S1 = gdr.gdr_chunk_fwd_ws(*x, S0, chunk=C)
    ws = gdr.gdr_chunk_intra(*x, chunk=C)
    o2, S2 = torch.empty_like(o1), torch.empty_like(S1)
    gdr.gdr_chunk_scan(ws, S0, o2, S2, B=B, H=H, T=T, dk=dk, dv=dv, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
