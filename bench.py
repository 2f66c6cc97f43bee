#!/usr/bin/env python3
"""Benchmark of the local graph-attention forward on one MI355X.

Workload: the 1M-node dot-product configuration -- N = 2^20 nodes, every node with
16 in-edges drawn uniformly plus one self-loop (E = 17 N = 17,825,792), H = 8 heads of
r = 64, q/k/v stored as bf16 (N(0,1) rounded to nearest even), fp32 accumulation and
fp32 output, score scale 1/sqrt(64).  A step is one fused forward pass (out and lse)
over the resident inputs; the CSR build and the degree plan are per-topology work and
are timed and reported separately.

Prints one JSON line with the throughput in GEdges/s, the roofline of the forward
kernel (algorithmic HBM bytes per launch over the launch time measured with HIP events
on the launch stream), and the CPU oracle timed on this host over the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s

# HBM bytes per forward launch counted by rocprofv3 (FETCH_SIZE x 2.00 + WRITE_SIZE x 1.00,
# factors from a plain 1 GiB copy) for the kernel as of the committed profile summary
# profiles/local_fwd_dot_n1m_h8_r64_bf16.md; None once the kernel changes.
COUNTED_TRAFFIC_GB = 39.95


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def fwd_bytes(n: int, e: int, heads: int, c: int, esz: int, with_lse: bool) -> int:
    """Algorithmic HBM bytes of one forward launch of the per-destination pull method:
    q once, one key row and one value row per edge, col per edge, row_ptr, out once,
    lse once."""
    w = heads * c
    b = n * w * esz + e * (2 * w * esz + 4) + 4 * (n + 1) + n * w * 4
    if with_lse:
        b += n * heads * 4
    return b


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures a single GPU; runs on more than one GPU are not part of this build",
              file=sys.stderr)
        return 2

    import torch

    import sparse_graph_attention_amd as g
    import synth

    ident = 3
    w = synth.WORKLOADS[ident]
    n, heads, c = w.n, w.heads, w.head_dim
    dev = torch.device("cuda:0")
    t0 = time.time()
    src, dst = synth.workload_graph(ident)
    e = int(src.size)
    log(f"workload {w.name}: n={n} e={e} H={heads} C={c} bf16 (graph {time.time() - t0:.1f}s)")
    bits = [synth.to_bf16_bits(synth.node_tensor(ident, i, (n, heads, c))) for i in range(3)]
    q, k, v = (torch.from_numpy(b.view(np.int16).reshape(n, heads, c)).to(dev).view(torch.bfloat16) for b in bits)
    src_d = torch.from_numpy(src).to(dev)
    dst_d = torch.from_numpy(dst).to(dev)
    log(f"inputs resident ({time.time() - t0:.1f}s)")

    stream = torch.cuda.current_stream()
    # per-topology work: CSR by destination and the degree plan
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    row_ptr, col, eid = g.gga_coo_to_csr(n, dst_d, src_d)
    ev[1].record(stream)
    plan = g.gga_plan_build(n, e, row_ptr)
    ev[2].record(stream)
    torch.cuda.synchronize()
    csr_ms, plan_ms = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])

    desc = g.make_desc(n, e, heads, c, g.GGA_SCORE_DOT, g.GGA_BF16, 1.0 / np.sqrt(c))
    out = torch.empty(n, heads, c, dtype=torch.float32, device=dev)
    lse = torch.empty(n, heads, dtype=torch.float32, device=dev)
    ws_bytes = g.lib.gga_local_attn_fwd_workspace(g.ctypes.byref(desc))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step():
        g.gga_local_attn_fwd(desc, q, k, v, row_ptr, col, plan, out=out, lse=lse, ws=ws)

    for _ in range(args.warmup):
        step()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    launch_ms = [s.elapsed_time(x) for s, x in zip(starts, ends)]
    ms_step = wall * 1e3 / args.steps
    kern_ms = float(np.mean(launch_ms))
    log(f"fwd: wall {ms_step:.3f} ms/step, launch avg {kern_ms:.3f} ms (min {min(launch_ms):.3f}, "
        f"max {max(launch_ms):.3f}); csr {csr_ms:.2f} ms, plan {plan_ms:.2f} ms")

    alg = fwd_bytes(n, e, heads, c, 2, True)
    achieved = alg / (kern_ms * 1e-3) / 1e9

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies done")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        hosts = [synth.bf16_bits_to_f32(b).reshape(n, heads, c).astype(np.float64) for b in bits]
        og = oracle.Graph(n, src, dst)
        t1 = time.perf_counter()
        oracle.local_fwd_dot(hosts[0], hosts[1], hosts[2], og, 1.0 / np.sqrt(c))
        dt = time.perf_counter() - t1
        cpu = {"value": e / dt / 1e9, "unit": "GEdges/s", "cores": oracle.threads(), "kind": "oracle",
               "sample": f"the whole forward of this workload ({e} edges, all {n} rows), fp64, {dt:.1f} s"}
        log(f"cpu oracle: {dt:.2f} s with {oracle.threads()} threads")

    rec = {
        "metric": "GEdges/s (x heads) for local graph-attention fwd; achieved HBM GB/s vs peak",
        "value": e / (ms_step * 1e-3) / 1e9,
        "unit": "GEdges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "nodes": n, "edges": e, "heads": heads, "head_dim": c,
                   "in_degree": "16 uniform + 1 self-loop", "storage": "bf16 q/k/v, fp32 out/lse",
                   "global_batch": 1, "seq_len": n, "parallelism": "single GPU"},
        "gedge_heads_per_s": e * heads / (ms_step * 1e-3) / 1e9,
        "hbm_gbs_algorithmic": achieved,
        "csr_build_ms": csr_ms,
        "plan_build_ms": plan_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": COUNTED_TRAFFIC_GB,
                     "kernel": "local_fwd_kernel (+ heavy-row merge launch)", "alg_bytes_per_launch": alg,
                     "launch_ms": kern_ms},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
