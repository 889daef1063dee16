"""Benchmark of the gated delta-rule hot path on one MI355X.

A step is one forward over the 4K-token workload through the two-kernel
entry points (``gdr_chunk_intra`` then ``gdr_chunk_scan``, which together
are ``gdr_chunk_fwd_ws``): B=4 sequences x H=16 heads x T=4096 tokens,
d_k = d_v = 128, chunk 64, bfloat16 inputs and outputs, float32 state,
S0 = 0, inputs resident in HBM. Inputs are seeded synthetic data with the
shapes and gate distributions of the Muir page's models (q, k = unit-norm
SiLU of N(0,1); v ~ N(0,1); alpha = sigmoid(N(4, 1.5)); b, w =
sigmoid(N(0,1))).

Printed: one JSON line with tokens/s (value); the path's roofline position
(the algorithmic bytes of the whole forward, 1,792 B per token-head plus the
final state, over the step time, against 8 TB/s) with the counter-measured
HBM traffic of its two kernels; each kernel's own compulsory bytes and
duration; the path's MFMA throughput against the bf16 peak; side legs for
the 32K-token workload, the fused single-kernel entry point, the decode step
(256 sequences, and 512 as a control whose state cannot sit in the 256 MB
last-level cache) and the mLSTM forward; and the float64 CPU oracle timed on
the host's cores over the whole 4K workload.
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
# the CPU share of one GPU on the benchmark hosts
HOST_CORE_SHARE = 16


def chunk_flops_per_chunk(C, dk, dv):
    """Algorithmic FLOPs of one chunk of one head: Gram L and M, the triangular
    solve, the three S0/state products and M V~."""
    return 2 * dk * C * C + C * (C - 1) * (dv + dk) + 6 * C * dk * dv + C * (C + 1) * dv


def chunk_bytes(B, H, T, dk, dv, es, s0=False, s_out=True):
    """Algorithmic HBM bytes of one chunkwise forward: q, k, alpha, b, v, w read
    once, o written once (input dtype), S0 read and S_T written (fp32)."""
    n = B * H * T
    b = n * (4 * dk + 2 * dv) * es + n * dv * es
    b += B * H * dk * dv * 4 * (int(s0) + int(s_out))
    return b


# The sources each measured kernel is compiled from (its file and the headers
# that file includes): a committed counter reading of that kernel stays valid
# until one of them changes.
KERNEL_SOURCES = {
    "chunk": ("gdr_chunk2.hip", "gdr_chunk_common.hpp", "gdr_device.hpp", "gdr_internal.h", "gdr_host.hpp",
              "gdr_record.hpp"),
    "chunk_fused": ("gdr_chunk.hip", "gdr_chunk_common.hpp", "gdr_device.hpp", "gdr_internal.h", "gdr_host.hpp"),
    "decode": ("gdr_decode.hip", "gdr_device.hpp", "gdr_internal.h"),
    "mlstm": ("gdr_mlstm2.hip", "gdr_device.hpp", "gdr_internal.h", "gdr_host.hpp"),
    "mlstm_fused": ("gdr_mlstm.hip", "gdr_device.hpp", "gdr_internal.h", "gdr_host.hpp"),
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


def load_traffic(launches_key):
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
    region, mean ms per launch). Events are recorded on torch's current
    stream, which the binding passes to the library."""
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


def chunk_inputs(name):
    import torch
    from synth import CONFIGS, gdn2_inputs
    c = CONFIGS[name]
    d = gdn2_inputs(c["B"], c["H"], c["T"], c["dk"], c["dv"], alpha_mu=c["alpha_mu"],
                    alpha_sigma=c["alpha_sigma"], seed=0, dtype="bf16", s0_std=c["s0_std"])
    x = [to_dev(d[n], torch.bfloat16) for n in ("q", "k", "v", "alpha", "b", "w")]
    S0 = None if d["S0"] is None else to_dev(d["S0"], torch.float32)
    return c, d, x, S0


def bench_chunk(steps, warmup, c, x, S0):
    """One step = gdr_chunk_intra then gdr_chunk_scan (= gdr_chunk_fwd_ws), with
    an event at every kernel boundary inside the timed region."""
    import torch
    import matrix_memory_rnn_amd as gdr
    B, H, T, dk, dv, C = c["B"], c["H"], c["T"], c["dk"], c["dv"], c["chunk"]
    o = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    nws = gdr.gdr_chunk_workspace_size(B, H, T, dk, dv, C, torch.bfloat16)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")

    def step():
        gdr.gdr_chunk_intra(*x, chunk=C, workspace=ws)
        gdr.gdr_chunk_scan(ws, S0, o, S, B=B, H=H, T=T, dk=dk, dv=dv, chunk=C)

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
        gdr.gdr_chunk_scan(ws, S0, o, S, B=B, H=H, T=T, dk=dk, dv=dv, chunk=C)
        bnd[i + 1].record()
    torch.cuda.synchronize()
    region = bnd[0].elapsed_time(bnd[-1]) / steps
    intra_ms = float(np.mean([bnd[i].elapsed_time(mid[i]) for i in range(steps)]))
    scan_ms = float(np.mean([mid[i].elapsed_time(bnd[i + 1]) for i in range(steps)]))
    n = B * H * T
    s0b = 0 if S0 is None else B * H * dk * dv * 4
    intra_bytes = n * (4 * dk + 2 * dv) * 2 + nws               # inputs read, workspace written
    scan_bytes = nws + n * dv * 2 + B * H * dk * dv * 4 + s0b     # workspace (+ S0) read, o and S_T written
    flops = chunk_flops_per_chunk(C, dk, dv) * (T // C) * B * H
    return dict(B=B, H=H, T=T, dk=dk, dv=dv, C=C, region_ms=region, intra_ms=intra_ms, scan_ms=scan_ms,
                intra_bytes=intra_bytes, scan_bytes=scan_bytes, ws_bytes=nws, flops=flops,
                bytes=chunk_bytes(B, H, T, dk, dv, 2, s0=S0 is not None))


def bench_fused(steps, warmup, c, x, S0):
    """The single-kernel entry point gdr_chunk_fwd on the same workload."""
    import torch
    import matrix_memory_rnn_amd as gdr
    B, H, T, dk, dv, C = c["B"], c["H"], c["T"], c["dk"], c["dv"], c["chunk"]
    o = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    fn = lambda: gdr.gdr_chunk_fwd(*x, S0, chunk=C, o=o, S_out=S)
    return time_launches(fn, steps, warmup)


def bench_muir(steps, warmup):
    """The Muir gate prologue on the 4K workload's shape: gdr_muir_chunk_fwd_ws
    reads q, k, v and the logits z_f, z_b, z_w, z_q (bf16) plus a_log and
    gamma_stat, and forms the gates inside the intra-chunk kernel."""
    import torch
    import matrix_memory_rnn_amd as gdr
    from synth import CONFIGS, muir_inputs
    c = CONFIGS["chunk_4k"]
    B, H, T, dk, dv, C = c["B"], c["H"], c["T"], c["dk"], c["dv"], c["chunk"]
    d = muir_inputs(B, H, T, dk, dv, seed=0, dtype="bf16")
    x = [to_dev(d[n], torch.bfloat16) for n in ("q", "k", "v", "z_f", "z_b", "z_w")]
    zq = to_dev(d["z_q"], torch.bfloat16)
    al, gs = to_dev(d["a_log"], torch.float32), to_dev(d["gamma_stat"], torch.float32)
    o = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdr.gdr_chunk_workspace_size(B, H, T, dk, dv, C, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    fn = lambda: gdr.gdr_muir_chunk_fwd_ws(*x, al, zq, gs, chunk=C, o=o, S_out=S, workspace=ws)
    region_ms, _ = time_launches(fn, steps, warmup)
    n = B * H * T
    nbytes = n * (5 * dk + 2 * dv) * 2 + n * dv * 2 + B * H * dk * dv * 4 + H * (dk + 1) * 4
    return dict(B=B, T=T, region_ms=region_ms, bytes=nbytes)


def bench_bwd(steps, warmup, c, x):
    """gdr_chunk_bwd on the 4K workload (bf16, S0 = 0, dS_T = 0): gradients
    of every input from dO, once recomputing the forward records and once
    from records the forward left in the workspace."""
    import torch
    import matrix_memory_rnn_amd as gdr
    B, H, T, dk, dv, C = c["B"], c["H"], c["T"], c["dk"], c["dv"], c["chunk"]
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    dO = torch.randn((B, H, T, dv), generator=g, device="cuda").to(torch.bfloat16)
    ws = torch.empty(gdr.gdr_chunk_bwd_workspace_size(B, H, T, dk, dv, C, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    gdr.gdr_chunk_intra(*x, chunk=C, workspace=ws)
    full, _ = time_launches(lambda: gdr.gdr_chunk_bwd(*x, None, dO, chunk=C, workspace=ws), steps, warmup)
    gdr.gdr_chunk_intra(*x, chunk=C, workspace=ws)
    ready, _ = time_launches(lambda: gdr.gdr_chunk_bwd(*x, None, dO, chunk=C, workspace=ws, records_ready=True),
                             steps, warmup)
    # algorithmic bytes: q, k, alpha, b, v, w, dO read (bf16), the six input
    # gradients written (fp32), dS0 written
    nbytes = B * H * T * ((4 * dk + 3 * dv) * 2 + (4 * dk + 2 * dv) * 4) + B * H * dk * dv * 4
    return dict(B=B, T=T, full_ms=full, ready_ms=ready, ws_bytes=ws.numel(), bytes=nbytes)


def bench_rwkv7(steps, warmup):
    """RWKV-7's generalized delta rule on the 4K workload's shape (B=4, H=16,
    T=4096, d=128, bf16, chunk 32) through gdr_rwkv7_fwd."""
    import torch
    import matrix_memory_rnn_amd as gdr
    from synth import CONFIGS, rwkv7_inputs
    c = CONFIGS["chunk_4k"]
    B, H, T, dk, dv = c["B"], c["H"], c["T"], c["dk"], c["dv"]
    d = rwkv7_inputs(B, H, T, dk, dv, seed=0, dtype="bf16")
    x = {n: to_dev(d[n], torch.bfloat16) for n in ("q", "w", "a", "kw", "u")}
    cc = to_dev(d["c"], torch.float32)
    o = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdr.gdr_rwkv7_workspace_size(B, H, T, dk, dv, 32), dtype=torch.uint8, device="cuda")
    fn = lambda: gdr.gdr_rwkv7_fwd(x["q"], x["w"], x["a"], cc, x["kw"], x["u"], chunk=32, o=o, S_out=S,
                                   workspace=ws)
    region_ms, _ = time_launches(fn, steps, warmup)
    nbytes = B * H * T * (4 * dk + 2 * dv) * 2 + B * H * T * 4 + B * H * dk * dv * 4
    return dict(B=B, T=T, region_ms=region_ms, bytes=nbytes)


def bench_decode(N, steps=1024):
    """N sequences x 16 heads, d = 128, fp32 states resident in HBM: `steps`
    sequential one-token updates, each with its own inputs (all `steps` input
    sets are drawn on the GPU before the timed region from a seeded
    generator, with the 4K workload's distributions)."""
    import torch
    import matrix_memory_rnn_amd as gdr
    H, dk, dv = 16, 128, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(0)

    def unit_silu(shape):
        z = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
        s = torch.nn.functional.silu(z)
        return (s / s.norm(dim=-1, keepdim=True)).to(torch.bfloat16)

    sh_k, sh_v = (steps, N, H, dk), (steps, N, H, dv)
    q, k = unit_silu(sh_k), unit_silu(sh_k)
    v = torch.randn(sh_v, generator=g, device="cuda").to(torch.bfloat16)
    a = torch.sigmoid(4.0 + 1.5 * torch.randn(sh_k, generator=g, device="cuda")).to(torch.bfloat16)
    b = torch.sigmoid(torch.randn(sh_k, generator=g, device="cuda")).to(torch.bfloat16)
    w = torch.sigmoid(torch.randn(sh_v, generator=g, device="cuda")).to(torch.bfloat16)
    S = torch.zeros((N, H, dk, dv), dtype=torch.float32, device="cuda")
    o = torch.empty((N, H, dv), dtype=torch.bfloat16, device="cuda")
    it = [0]

    def fn():
        i = it[0] % steps
        gdr.gdr_decode_step(q[i], k[i], v[i], a[i], b[i], w[i], S, o=o)
        it[0] += 1

    for _ in range(16):
        fn()
    S.zero_()
    it[0] = 0
    region_ms, launch_ms = time_launches(fn, steps, 0)
    nbytes = 2 * N * H * dk * dv * 4 + N * H * (4 * dk + 2 * dv) * 2 + N * H * dv * 2
    del q, k, v, a, b, w
    return dict(N=N, H=H, steps=steps, region_ms=region_ms, launch_ms=launch_ms, bytes=nbytes)


def bench_mlstm(steps, warmup):
    """mLSTM forward on the 8K workload (B=2, H=8, T=8192, d=256, C=64, bf16),
    returning h and the final (C, n, m): the two-kernel entry point
    gdr_mlstm_fwd_ws and the fused gdr_mlstm_fwd."""
    import torch
    import matrix_memory_rnn_amd as gdr
    from synth import CONFIGS, mlstm_inputs
    c = CONFIGS["mlstm_8k"]
    B, H, T, dk, dv, C = c["B"], c["H"], c["T"], c["dk"], c["dv"], c["chunk"]
    d = mlstm_inputs(B, H, T, dk, dv, seed=0, dtype="bf16")
    q, k, v = (to_dev(d[n], torch.bfloat16) for n in ("q", "k", "v"))
    it, ft = (to_dev(d[n], torch.float32) for n in ("i_tilde", "f_tilde"))
    h = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device="cuda")
    Co = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    no = torch.empty((B, H, dk), dtype=torch.float32, device="cuda")
    mo = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdr.gdr_mlstm_workspace_size(B, H, T, dk, dv, C, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    out = dict(h=h, C_out=Co, n_out=no, m_out=mo)
    fn_ws = lambda: gdr.gdr_mlstm_fwd_ws(q, k, v, it, ft, chunk=C, workspace=ws, **out)
    fn_f = lambda: gdr.gdr_mlstm_fwd(q, k, v, it, ft, chunk=C, **out)
    region_ms, launch_ms = time_launches(fn_ws, steps, warmup)
    fused_ms, _ = time_launches(fn_f, steps, warmup)
    nbytes = B * H * T * (2 * dk + 2 * dv) * 2 + B * H * T * 8 + B * H * (dk * dv + dk + 1) * 4
    flops_chunk = C * (C + 1) * dk + C * (C + 1) * (dv + 1) + 4 * C * dk * (dv + 1)
    flops = flops_chunk * (T // C) * B * H
    return dict(B=B, H=H, T=T, region_ms=region_ms, launch_ms=launch_ms, fused_ms=fused_ms, bytes=nbytes,
                ws_bytes=ws.numel(), flops=flops)


def _oracle_heads(args):
    """CPU worker: the float64 oracle on a slice of heads (one thread)."""
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t = time.perf_counter()
        oracle.gdn2_recurrent(*args)
        return time.perf_counter() - t


def cpu_baseline(d):
    """The float64 oracle over the whole 4K workload (4 x 16 heads x 4096
    tokens), its heads split over a pool of single-threaded worker processes,
    one per host core of the GPU's share."""
    import concurrent.futures as cf
    import multiprocessing as mp
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    workers = max(1, min(HOST_CORE_SHARE, avail))
    names = ("q", "k", "v", "alpha", "b", "w")
    B, H, T = d["q"].shape[:3]
    heads = [(b, h) for b in range(B) for h in range(H)]
    parts = [heads[i::workers] for i in range(workers)]
    jobs = []
    for p in parts:
        if not p:
            continue
        bi, hi = np.array([x[0] for x in p]), np.array([x[1] for x in p])
        jobs.append(tuple(np.ascontiguousarray(d[n][bi, hi][None]) for n in names))
    # fresh interpreters (no GPU runtime inherited); a worker that dies raises
    # BrokenProcessPool instead of being replaced
    with cf.ProcessPoolExecutor(max_workers=len(jobs), mp_context=mp.get_context("spawn")) as pool:
        list(pool.map(_oracle_heads, jobs[:1]))          # start-up outside the timed region
        t = time.perf_counter()
        busy = list(pool.map(_oracle_heads, jobs))
        wall = time.perf_counter() - t
    return {"value": B * T / wall, "unit": "tokens/s", "cores": len(jobs), "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "host_cores_available": avail,
            "sample": f"the whole workload ({B} x {H} heads x {T} tokens), float64 numpy, heads split over "
                      f"{len(jobs)} single-threaded processes: {wall:.2f} s wall, {sum(busy):.1f} s of CPU work"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-side", action="store_true", help="skip every leg but the 4K chunk forward")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB elementwise copy (dst = src * 1) three times: the "
                         "known-size kernel that calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: every (sequence, head) pair is independent, so a batch "
              "shards across GPUs with no communication, and nothing here runs on more than one. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    c, d, x, S0 = chunk_inputs("chunk_4k")
    r = bench_chunk(args.steps, args.warmup, c, x, S0)
    tokens = r["B"] * r["T"]
    value = tokens / (r["region_ms"] * 1e-3)
    kern = {
        "intra": {"ms": r["intra_ms"], "bytes": r["intra_bytes"],
                  "GB/s": r["intra_bytes"] / (r["intra_ms"] * 1e-3) / 1e9,
                  "traffic": load_traffic("chunk_intra_4k")},
        "scan": {"ms": r["scan_ms"], "bytes": r["scan_bytes"],
                 "GB/s": r["scan_bytes"] / (r["scan_ms"] * 1e-3) / 1e9,
                 "traffic": load_traffic("chunk_scan_4k")},
    }
    for v in kern.values():
        v["frac_hbm"] = v["GB/s"] / PEAK_HBM_GBS
        v["note"] = "kernel-level: the kernel's own compulsory bytes (workspace included) over its duration"
    path_gbs = r["bytes"] / (r["region_ms"] * 1e-3) / 1e9
    tflops = r["flops"] / (r["region_ms"] * 1e-3) / 1e12
    traffic = None
    if kern["intra"]["traffic"] is not None and kern["scan"]["traffic"] is not None:
        traffic = kern["intra"]["traffic"] + kern["scan"]["traffic"]
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
        "roofline": {"bound": "hbm", "kernel": "gdn2_chunk_intra + gdn2_chunk_scan (the whole forward)",
                     "achieved": path_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": path_gbs / PEAK_HBM_GBS, "traffic": traffic,
                     "algorithmic_bytes": r["bytes"], "units": f"{tokens * r['H']} token-heads x 1792 B "
                     f"+ {r['B'] * r['H']} final states x 64 KiB",
                     "ms": r["region_ms"], "hbm_floor_ms": r["bytes"] / (PEAK_HBM_GBS * 1e9) * 1e3,
                     "workspace_bytes": r["ws_bytes"]},
        "mfma": {"tflops": tflops, "peak": PEAK_BF16_TFLOPS, "frac": tflops / PEAK_BF16_TFLOPS,
                 "flops_per_step": r["flops"],
                 "ceiling_frac_at_hbm_floor": r["flops"] / (r["bytes"] / (PEAK_HBM_GBS * 1e9)) / 1e12
                 / PEAK_BF16_TFLOPS,
                 "note": "algorithmic FLOPs of the path (masked tiles not counted)"},
        "kernels": kern,
        "token_heads_per_s": value * r["H"],
    }
    if not args.no_side:
        bw = bench_bwd(max(10, args.steps // 4), max(3, args.warmup // 10), c, x)
        out["backward"] = {"workload": "4K workload, gradients of q, k, v, alpha, b, w and S0 from dO",
                           "entry": "gdr_chunk_bwd", "ms_per_step": bw["full_ms"],
                           "ms_per_step_records_ready": bw["ready_ms"],
                           "tokens/s": bw["B"] * bw["T"] / (bw["full_ms"] * 1e-3), "workspace_bytes": bw["ws_bytes"],
                           "algorithmic_bytes": bw["bytes"], "GB/s": bw["bytes"] / (bw["full_ms"] * 1e-3) / 1e9,
                           "frac_hbm": bw["bytes"] / (bw["full_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del x
    if not args.no_side:
        f_region, f_launch = bench_fused(args.steps, args.warmup, c, chunk_inputs("chunk_4k")[2], None)
        fb = r["bytes"] / (f_region * 1e-3) / 1e9
        out["fused"] = {"entry": "gdr_chunk_fwd (one kernel, no workspace), 4K workload", "ms_per_step": f_region,
                        "kernel_ms": f_launch, "tokens/s": tokens / (f_region * 1e-3), "GB/s": fb,
                        "frac_hbm": fb / PEAK_HBM_GBS}
        mu = bench_muir(args.steps, args.warmup)
        mg = mu["bytes"] / (mu["region_ms"] * 1e-3) / 1e9
        out["muir_prologue"] = {"workload": "4K workload shape with gate logits: q, k, v, z_f, z_b, z_w, z_q bf16, "
                                            "a_log [H], gamma_stat [H, dk]",
                                "entry": "gdr_muir_chunk_fwd_ws", "ms_per_step": mu["region_ms"],
                                "tokens/s": mu["B"] * mu["T"] / (mu["region_ms"] * 1e-3),
                                "algorithmic_bytes": mu["bytes"], "GB/s": mg, "frac_hbm": mg / PEAK_HBM_GBS}
        r7 = bench_rwkv7(max(10, args.steps // 4), max(3, args.warmup // 10))
        g7 = r7["bytes"] / (r7["region_ms"] * 1e-3) / 1e9
        out["rwkv7"] = {"workload": "4K workload shape, RWKV-7 generalized delta rule, bf16, chunk 32",
                        "entry": "gdr_rwkv7_fwd", "ms_per_step": r7["region_ms"],
                        "tokens/s": r7["B"] * r7["T"] / (r7["region_ms"] * 1e-3), "GB/s": g7,
                        "frac_hbm": g7 / PEAK_HBM_GBS}
        c3, _, x3, S03 = chunk_inputs("chunk_32k")
        r3 = bench_chunk(max(10, args.steps // 4), max(5, args.warmup // 4), c3, x3, S03)
        g3 = r3["bytes"] / (r3["region_ms"] * 1e-3) / 1e9
        out["chunk_32k"] = {"workload": "gdn2 chunk fwd B=1 H=16 T=32768 d=128 C=64, bf16, S0~N(0,0.02)",
                            "entry": "gdr_chunk_intra + gdr_chunk_scan", "ms_per_step": r3["region_ms"],
                            "intra_ms": r3["intra_ms"], "scan_ms": r3["scan_ms"],
                            "tokens/s": r3["B"] * r3["T"] / (r3["region_ms"] * 1e-3),
                            "algorithmic_bytes": r3["bytes"], "GB/s": g3, "frac_hbm": g3 / PEAK_HBM_GBS,
                            "mfma_frac": r3["flops"] / (r3["region_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        del x3, S03
        for N, key in ((256, "decode"), (512, "decode_512")):
            dd = bench_decode(N)
            gbs = dd["bytes"] / (dd["launch_ms"] * 1e-3) / 1e9
            out[key] = {"workload": f"{N} seq x 16 heads, d=128, fp32 state ({N * 16 * 64 // 1024} MiB), "
                                    f"1024 steps, fresh inputs each step",
                        "ms_per_step": dd["region_ms"], "kernel_ms": dd["launch_ms"], "GB/s": gbs,
                        "frac_hbm": gbs / PEAK_HBM_GBS, "tokens/s": dd["N"] / (dd["region_ms"] * 1e-3),
                        "traffic": load_traffic("decode_256x16") if N == 256 else None}
            torch.cuda.empty_cache()
        mm = bench_mlstm(args.steps, args.warmup)
        mt = mm["B"] * mm["T"] / (mm["region_ms"] * 1e-3)
        mg = mm["bytes"] / (mm["region_ms"] * 1e-3) / 1e9
        out["mlstm"] = {"workload": "B=2 H=8 T=8192 d=256 C=64 bf16, h and final (C, n, m) returned",
                        "entry": "gdr_mlstm_fwd_ws", "ms_per_step": mm["region_ms"], "tokens/s": mt,
                        "algorithmic_bytes": mm["bytes"], "GB/s": mg, "frac_hbm": mg / PEAK_HBM_GBS,
                        "mfma_frac": mm["flops"] / (mm["region_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
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
