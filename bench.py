"""Benchmark of the gated delta-rule hot path on one MI355X.

A step is one forward over the 4K-token workload through the two-kernel
entry points (``gdr_chunk_intra`` then ``gdr_chunk_scan``, which together
are ``gdr_chunk_fwd_ws``):
B=4 sequences x H=16 heads x T=4096 tokens, d_k = d_v = 128, chunk 64,
bfloat16 inputs and outputs, float32 state, S0 = 0, inputs resident in HBM.
Inputs are seeded synthetic data with the shapes and gate distributions of
the Muir page's models (q, k = unit-norm SiLU of N(0,1); v ~ N(0,1);
alpha = sigmoid(N(4, 1.5)); b, w = sigmoid(N(0,1))).

Printed: one JSON line with tokens/s (value); the roofline position of the
dominant kernel (HBM-bound; its compulsory bytes per launch over its mean
event-timed duration) and of each kernel; the path's algorithmic bytes and
MFMA throughput against the MI355X peaks; side measurements for the fused
single-kernel entry point, the decode step (HBM GB/s) and the mLSTM forward;
and the float64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2516.6


def chunk_flops_per_chunk(C, dk, dv):
    """Algorithmic FLOPs of one chunk of one head: Gram L and M, the triangular
    solve, the three S0/state products and M V~."""
    return 2 * dk * C * C + C * (C - 1) * (dv + dk) + 6 * C * dk * dv + C * (C + 1) * dv


def chunk_bytes(B, H, T, dk, dv, es, s0=False, s_out=True):
    n = B * H * T
    b = n * (4 * dk + 2 * dv) * es + n * dv * es
    b += B * H * dk * dv * 4 * (int(s0) + int(s_out))
    return b


# The sources each measured kernel is compiled from (its file and the headers
# that file includes): a committed counter reading of that kernel stays valid
# until one of them changes.
KERNEL_SOURCES = {
    "chunk": ("gdr_chunk2.hip", "gdr_chunk_common.hpp", "gdr_device.hpp", "gdr_internal.h"),
    "chunk_fused": ("gdr_chunk.hip", "gdr_chunk_common.hpp", "gdr_device.hpp", "gdr_internal.h"),
    "decode": ("gdr_decode.hip", "gdr_device.hpp", "gdr_internal.h"),
    "mlstm": ("gdr_mlstm2.hip", "gdr_device.hpp", "gdr_internal.h"),
    "mlstm_fused": ("gdr_mlstm.hip", "gdr_device.hpp", "gdr_internal.h"),
}
COUNTER_KEYS = {"chunk_intra_4k": "chunk", "chunk_scan_4k": "chunk", "chunk_fwd_4k": "chunk_fused",
                "decode_256x16": "decode", "mlstm_intra_8k": "mlstm", "mlstm_scan_8k": "mlstm",
                "mlstm_fused_8k": "mlstm_fused"}


def kernel_source_hash(group):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "matrix_memory_rnn_amd", "csrc")
    for f in KERNEL_SOURCES[group]:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(name, launches_key):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or None
    when missing or taken on different kernel sources."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        data = json.load(f)
    e = data.get(launches_key)
    if not e or e.get("source_hash") != kernel_source_hash(COUNTER_KEYS[launches_key]):
        return None
    return e.get("hbm_bytes_per_launch")


def to_dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32)
    return t.to(dtype).cuda()


def time_launches(fn, steps, warmup):
    """Run fn warmup times, then `steps` times with one event between
    consecutive launches (launch i runs from event i to event i + 1, so the
    region is exactly the sum of the launches); returns (ms per step over the
    region, mean ms per launch)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    bnd = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    bnd[0].record()
    for i in range(steps):
        fn()
        bnd[i + 1].record()
    torch.cuda.synchronize()
    per = [bnd[i].elapsed_time(bnd[i + 1]) for i in range(steps)]
    return bnd[0].elapsed_time(bnd[-1]) / steps, float(np.mean(per))


def chunk_inputs():
    import torch
    from synth import CONFIGS, gdn2_inputs
    c = CONFIGS["chunk_4k"]
    d = gdn2_inputs(c["B"], c["H"], c["T"], c["dk"], c["dv"], alpha_mu=c["alpha_mu"],
                    alpha_sigma=c["alpha_sigma"], seed=0, dtype="bf16")
    x = [to_dev(d[n], torch.bfloat16) for n in ("q", "k", "v", "alpha", "b", "w")]
    return c, d, x


def bench_chunk(steps, warmup, c, x):
    """One step = gdr_chunk_intra then gdr_chunk_scan (= gdr_chunk_fwd_ws) on
    the 4K workload, with an event at every kernel boundary inside the timed
    region."""
    import torch
    import matrix_memory_rnn_amd as gdr
    B, H, T, dk, dv, C = c["B"], c["H"], c["T"], c["dk"], c["dv"], c["chunk"]
    o = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    nws = gdr.gdr_chunk_workspace_size(B, H, T, dk, dv, C, torch.bfloat16)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")

    def step():
        gdr.gdr_chunk_intra(*x, chunk=C, workspace=ws)
        gdr.gdr_chunk_scan(ws, None, o, S, B=B, H=H, T=T, dk=dk, dv=dv, chunk=C)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # one event at each step boundary and one between the two kernels: the
    # intra kernel of step i runs from bnd[i] to mid[i], its scan from mid[i]
    # to bnd[i + 1], and the region is exactly the sum of the kernels
    bnd = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    mid = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    bnd[0].record()
    for i in range(steps):
        gdr.gdr_chunk_intra(*x, chunk=C, workspace=ws)
        mid[i].record()
        gdr.gdr_chunk_scan(ws, None, o, S, B=B, H=H, T=T, dk=dk, dv=dv, chunk=C)
        bnd[i + 1].record()
    torch.cuda.synchronize()
    region = bnd[0].elapsed_time(bnd[-1]) / steps
    intra_ms = float(np.mean([bnd[i].elapsed_time(mid[i]) for i in range(steps)]))
    scan_ms = float(np.mean([mid[i].elapsed_time(bnd[i + 1]) for i in range(steps)]))
    n = B * H * T
    intra_bytes = n * (4 * dk + 2 * dv) * 2 + nws          # inputs read, workspace written
    scan_bytes = nws + n * dv * 2 + B * H * dk * dv * 4       # workspace read, o and S_T written
    flops = chunk_flops_per_chunk(C, dk, dv) * (T // C) * B * H
    return dict(B=B, H=H, T=T, dk=dk, dv=dv, C=C, region_ms=region, intra_ms=intra_ms, scan_ms=scan_ms,
                intra_bytes=intra_bytes, scan_bytes=scan_bytes, ws_bytes=nws, flops=flops,
                bytes=chunk_bytes(B, H, T, dk, dv, 2))


def bench_fused(steps, warmup, c, x):
    """The single-kernel entry point gdr_chunk_fwd on the same workload."""
    import torch
    import matrix_memory_rnn_amd as gdr
    B, H, T, dk, dv, C = c["B"], c["H"], c["T"], c["dk"], c["dv"], c["chunk"]
    o = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    fn = lambda: gdr.gdr_chunk_fwd(*x, None, chunk=C, o=o, S_out=S)
    return time_launches(fn, steps, warmup)


def bench_decode(steps=1024):
    """256 sequences x 16 heads, d = 128, fp32 states resident in HBM, `steps`
    sequential one-token updates with fresh inputs each step (drawn on the GPU
    from a seeded generator with the 4K workload's distributions)."""
    import torch
    import matrix_memory_rnn_amd as gdr
    N, H, dk, dv = 256, 16, 128, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    pool = 16

    def unit_silu(shape):
        z = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
        s = torch.nn.functional.silu(z)
        return (s / s.norm(dim=-1, keepdim=True)).to(torch.bfloat16)

    inp = []
    for _ in range(pool):
        q, k = unit_silu((N, H, dk)), unit_silu((N, H, dk))
        v = torch.randn((N, H, dv), generator=g, device="cuda").to(torch.bfloat16)
        a = torch.sigmoid(4.0 + 1.5 * torch.randn((N, H, dk), generator=g, device="cuda")).to(torch.bfloat16)
        b = torch.sigmoid(torch.randn((N, H, dk), generator=g, device="cuda")).to(torch.bfloat16)
        w = torch.sigmoid(torch.randn((N, H, dv), generator=g, device="cuda")).to(torch.bfloat16)
        inp.append((q, k, v, a, b, w))
    S = torch.zeros((N, H, dk, dv), dtype=torch.float32, device="cuda")
    o = torch.empty((N, H, dv), dtype=torch.bfloat16, device="cuda")
    it = [0]

    def fn():
        gdr.gdr_decode_step(*inp[it[0] % pool], S, o=o)
        it[0] += 1

    region_ms, launch_ms = time_launches(fn, steps, 16)
    nbytes = 2 * N * H * dk * dv * 4 + N * H * (4 * dk + 2 * dv) * 2 + N * H * dv * 2
    return dict(N=N, H=H, steps=steps, region_ms=region_ms, launch_ms=launch_ms, bytes=nbytes)


def bench_mlstm(steps, warmup):
    """mLSTM forward on the 8K workload (B=2, H=8, T=8192, d=256, C=64, bf16):
    the two-kernel entry point gdr_mlstm_fwd_ws and the fused gdr_mlstm_fwd."""
    import torch
    import matrix_memory_rnn_amd as gdr
    from synth import CONFIGS, mlstm_inputs
    c = CONFIGS["mlstm_8k"]
    B, H, T, dk, dv, C = c["B"], c["H"], c["T"], c["dk"], c["dv"], c["chunk"]
    d = mlstm_inputs(B, H, T, dk, dv, seed=0, dtype="bf16")
    q, k, v = (to_dev(d[n], torch.bfloat16) for n in ("q", "k", "v"))
    it, ft = (to_dev(d[n], torch.float32) for n in ("i_tilde", "f_tilde"))
    h = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdr.gdr_mlstm_workspace_size(B, H, T, dk, dv, C, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    fn_ws = lambda: gdr.gdr_mlstm_fwd_ws(q, k, v, it, ft, chunk=C, h=h, return_state=False, workspace=ws)
    fn_f = lambda: gdr.gdr_mlstm_fwd(q, k, v, it, ft, chunk=C, h=h, return_state=False)
    region_ms, launch_ms = time_launches(fn_ws, steps, warmup)
    fused_ms, _ = time_launches(fn_f, steps, warmup)
    nbytes = B * H * T * (2 * dk + 2 * dv) * 2 + B * H * T * 8
    return dict(B=B, H=H, T=T, region_ms=region_ms, launch_ms=launch_ms, fused_ms=fused_ms, bytes=nbytes,
                ws_bytes=ws.numel())


def cpu_baseline(d):
    """The float64 oracle on one sequence (b = 0, all 16 heads, 4096 tokens) of
    the 4K workload, single-threaded."""
    import oracle
    from threadpoolctl import threadpool_limits
    sl = lambda x: np.ascontiguousarray(d[x][0:1])
    args = [sl(x) for x in ("q", "k", "v", "alpha", "b", "w")]
    with threadpool_limits(limits=1):
        t = time.perf_counter()
        oracle.gdn2_recurrent(*args)
        dt = time.perf_counter() - t
    T = args[0].shape[2]
    return {"value": T / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"b=0 of the 4K workload: 16 heads x {T} tokens, float64 numpy, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-side", action="store_true", help="skip the decode and mLSTM side measurements")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB elementwise copy (dst = src * 1) three times: the "
                         "known-size kernel that calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(batch/head sharding needs no communication; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    c, d, x = chunk_inputs()
    r = bench_chunk(args.steps, args.warmup, c, x)
    tokens = r["B"] * r["T"]
    value = tokens / (r["region_ms"] * 1e-3)
    kern = {
        "intra": {"ms": r["intra_ms"], "bytes": r["intra_bytes"],
                  "GB/s": r["intra_bytes"] / (r["intra_ms"] * 1e-3) / 1e9,
                  "traffic": load_traffic("intra", "chunk_intra_4k")},
        "scan": {"ms": r["scan_ms"], "bytes": r["scan_bytes"],
                 "GB/s": r["scan_bytes"] / (r["scan_ms"] * 1e-3) / 1e9,
                 "traffic": load_traffic("scan", "chunk_scan_4k")},
    }
    for v in kern.values():
        v["frac_hbm"] = v["GB/s"] / PEAK_HBM_GBS
    dom = max(kern, key=lambda k: kern[k]["ms"])
    path_gbs = r["bytes"] / (r["region_ms"] * 1e-3) / 1e9
    tflops = r["flops"] / (r["region_ms"] * 1e-3) / 1e12
    out = {
        "metric": "tokens/s + % bf16 MFMA peak, chunk fwd H=16 d=128 T=4K; decode HBM GB/s",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["region_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; gate distributions of the Muir page's models)",
        "config": {"workload": "gdn2 chunk fwd B=4 H=16 T=4096 dk=dv=128 C=64, bf16 in/out, fp32 state, S0=0",
                   "global_batch": r["B"], "seq_len": r["T"], "heads": r["H"], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": f"gdn2_chunk_{dom}", "achieved": kern[dom]["GB/s"],
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": kern[dom]["frac_hbm"],
                     "traffic": kern[dom]["traffic"], "bytes_per_launch": kern[dom]["bytes"]},
        "kernels": kern,
        "path": {"algorithmic_bytes": r["bytes"], "GB/s": path_gbs, "frac_hbm": path_gbs / PEAK_HBM_GBS,
                 "hbm_floor_ms": r["bytes"] / (PEAK_HBM_GBS * 1e9) * 1e3, "workspace_bytes": r["ws_bytes"]},
        "mfma": {"tflops": tflops, "peak": PEAK_BF16_TFLOPS, "frac": tflops / PEAK_BF16_TFLOPS,
                 "flops_per_step": r["flops"], "note": "algorithmic FLOPs of the path (masked tiles not counted)"},
        "token_heads_per_s": value * r["H"],
    }
    if not args.no_side:
        f_region, f_launch = bench_fused(args.steps, args.warmup, c, x)
        out["fused"] = {"entry": "gdr_chunk_fwd (one kernel, no workspace)", "ms_per_step": f_region,
                        "kernel_ms": f_launch, "tokens/s": tokens / (f_region * 1e-3)}
        dd = bench_decode()
        gbs = dd["bytes"] / (dd["launch_ms"] * 1e-3) / 1e9
        out["decode"] = {"workload": "256 seq x 16 heads, d=128, fp32 state, 1024 steps", "ms_per_step": dd["region_ms"],
                         "kernel_ms": dd["launch_ms"], "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS,
                         "tokens/s": dd["N"] / (dd["region_ms"] * 1e-3)}
        mm = bench_mlstm(args.steps, args.warmup)
        mt = mm["B"] * mm["T"] / (mm["region_ms"] * 1e-3)
        mg = mm["bytes"] / (mm["region_ms"] * 1e-3) / 1e9
        out["mlstm"] = {"workload": "B=2 H=8 T=8192 d=256 C=64 bf16", "entry": "gdr_mlstm_fwd_ws",
                        "ms_per_step": mm["region_ms"], "tokens/s": mt,
                        "algorithmic_bytes": mm["bytes"], "GB/s": mg, "frac_hbm": mg / PEAK_HBM_GBS,
                        "workspace_bytes": mm["ws_bytes"], "fused_ms_per_step": mm["fused_ms"]}
    if args.calib_copy:
        n = 64 * 1024 * 1024  # 256 MiB of float32 read, 256 MiB written per launch
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        out["calib_copy_bytes_each_way"] = n * 4
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
