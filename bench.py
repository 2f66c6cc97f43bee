#!/usr/bin/env python3
"""Benchmark of neighbor-restricted graph attention on one MI355X.

Default workload (the headline): the 1M-node dot-product configuration -- N = 2^20
nodes, each with 16 in-edges drawn uniformly plus one self-loop (E = 17 N =
17,825,792), H = 8 heads of r = 64, q/k/v stored as bf16 (N(0,1) rounded to nearest
even), fp32 accumulation and fp32 output, score scale 1/sqrt(64).  A step is one fused
forward pass (out and lse) over inputs already resident in HBM.  The CSR build and the
degree plan are per-topology work, timed and reported separately.

Other workloads (``--workload``), each printed as its own line when asked for:
  5  heavy-tailed 2M-node graph, H = 8, C = 32, bf16: a step is forward + backward
     (dQ over the CSR by destination, dK and dV over the CSR by source)
  2  170k-node power-law GAT layer, Fin = 128 -> 8 heads x 8, fp32: a step is the
     layer forward + its first-order gradients (dX, dW, da_s, da_t)
  4  262k-node gated local-global layer, d = 256, 4 heads of 64, fp32: a step is the
     layer forward + the gradients of every input and parameter
  6  the same layer over a batch of 64 graphs of 4096 nodes packed along the node axis
     (block-diagonal edges, per-graph global statistics): forward + gradients
  7  the 170k-node GAT layer with 16 learned features per edge in the score and the
     heads averaged: forward + first-order gradients
  8  relation-typed messages over 512 packed sequences of 256 tokens, d = 512, 8 heads of
     64, 3 relations, mean weighting: forward + gradients of the input and transforms
  9  the same with softmax weighting (shared query, per-relation keys and messages)
  1  tiny 1024-node dot-product graph, H = 1, r = 16, fp32: forward

Prints one JSON line: throughput in GEdges/s, the roofline of the dominant kernel call
(algorithmic HBM bytes per launch over the launch time measured with HIP events on the
launch stream) and the CPU oracle timed on this host over the same work.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
MFMA_F32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix

# HBM traffic counted by rocprofv3 (FETCH_SIZE x 2.00 + WRITE_SIZE x 1.00 per launch, the factors
# measured on a plain 1 GiB copy in the same runs), in GB per launch or call.  Each figure names
# the profile summary it comes from and a digest of the sources of the kernels it counted; it is
# reported only while those sources are unchanged (a changed kernel gets null traffic until its
# counters are taken again).
KERNEL_SOURCES = {
    "fwd": ["local_fwd.hip", "rowgeo.hpp", "shape.hpp", "plan.hpp", "common.hpp"],
    "bwd": ["local_bwd.hip", "local_bwd_impl.hpp", "local_bwd_bf16.hip", "local_bwd_f32.hip", "rowgeo.hpp",
            "shape.hpp", "plan.hpp", "common.hpp"],
}
COUNTED = {
    "fwd_w3": {"gb": 39.86, "profile": "profiles/local_fwd_dot_n1m_h8_r64_bf16.md", "sources": "fwd",
               "digest": "0f70097d25f36865"},
    "fwd_w5": {"gb": 72.56, "profile": "profiles/local_fwd_bwd_dot_n2m_zipf_h8_c32_bf16.md", "sources": "fwd",
               "digest": "0f70097d25f36865"},
    "bwd_w5": {"gb": 157.63, "profile": "profiles/local_fwd_bwd_dot_n2m_zipf_h8_c32_bf16.md", "sources": "bwd",
               "digest": "94fbeb65e5cdd369"},
    "bwd_w4": {"gb": 39.69, "profile": "profiles/gated_layer_n262k_d256_h4.md", "sources": "bwd",
               "digest": "94fbeb65e5cdd369"},
}


def sources_digest(kind: str) -> str:
    """sha256 (first 16 hex digits) over the named kernel sources, file name and bytes."""
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        h.update(name.encode())
        with open(os.path.join(ROOT, "sparse_graph_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counted_traffic(key: str):
    """The counted GB of COUNTED[key] while its kernel sources are unchanged, else None."""
    c = COUNTED[key]
    if c["gb"] is None or c["digest"] != sources_digest(c["sources"]):
        return None
    return c["gb"]


METRIC = "GEdges/s (x heads) for local graph-attention fwd; achieved HBM GB/s vs peak"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def fwd_bytes(n, e, heads, c, esz, with_lse=True) -> int:
    """Forward, per launch: q once, one key row and one value row per edge, col per edge,
    row_ptr, out once (fp32), lse once (fp32)."""
    w = heads * c
    return n * w * esz + e * (2 * w * esz + 4) + 4 * (n + 1) + n * w * 4 + (n * heads * 4 if with_lse else 0)


def bwd_bytes(n, e, heads, c, esz) -> int:
    """Backward, per call.  Pass A (CSR by destination): per edge a key and a value row and
    col; per node q, dO, out, lse, row_ptr, and dq and D written.  Pass B (CSR by source):
    per edge a query row, a dO row, lse and D of the target, and col; per node k, v,
    row_ptr, and dk, dv written."""
    w = heads * c
    a = e * (2 * w * esz + 4) + n * (w * esz + 8 * w + 4 * heads + 4) + n * (4 * w + 4 * heads)
    b = e * (w * esz + 4 * w + 8 * heads + 4) + n * (2 * w * esz + 4) + n * 8 * w
    return a + b


class Timer:
    """Times `steps` calls of step() after `warmup` untimed ones: wall clock between two
    device synchronisations, plus HIP events (on the launch stream) around named phases."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.events = {}

    def mark(self, name):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record(self.stream)
        self.events.setdefault(name, []).append(ev)

    def run(self, step, steps, warmup):
        for _ in range(warmup):
            step(None)
        self.events = {}
        self.torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            step(self)
        self.torch.cuda.synchronize()
        wall = (time.perf_counter() - t) * 1e3 / steps
        return wall

    def phase_ms(self, a, b):
        return float(np.mean([x.elapsed_time(y) for x, y in zip(self.events[a], self.events[b])]))

    def phase_median_ms(self, a, b):
        return float(np.median([x.elapsed_time(y) for x, y in zip(self.events[a], self.events[b])]))


def mall_cold_ms(torch, launch, reps, dev):
    """Launch times (HIP events around the launch) with a 1 GiB fill kernel run before each,
    so that the 256 MB MALL holds none of the inputs when the launch starts."""
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    out = []
    for _ in range(reps):
        scratch.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        launch()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    del scratch
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _mark(tm, name):
    if tm is not None:
        tm.mark(name)


TOPOLOGY_REPS = 10  # builds timed back to back (mean reported)


def per_topology(g, torch, n, src_d, dst_d, backward=False):
    # one untimed build first, so the timed ones see loaded kernels and a warm allocator
    g.Topology(n, src_d, dst_d, backward=backward)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(TOPOLOGY_REPS):
        row_ptr, col, eid = g.gga_coo_to_csr(n, dst_d, src_d)
    ev[1].record()
    for _ in range(TOPOLOGY_REPS):
        plan = g.gga_plan_build(n, int(src_d.numel()), row_ptr)
    ev[2].record()
    topo = g.Topology.__new__(g.Topology)
    topo.n, topo.n_src, topo.e, topo.src, topo.dst = n, n, int(src_d.numel()), src_d, dst_d
    topo.row_ptr, topo.col, topo.eid, topo.plan = row_ptr, col, eid, plan
    topo.row_ptr_s = topo.col_s = topo.eid_s = topo.plan_s = None
    torch.cuda.synchronize()
    t = {"csr_build_ms": ev[0].elapsed_time(ev[1]) / TOPOLOGY_REPS,
         "plan_build_ms": ev[1].elapsed_time(ev[2]) / TOPOLOGY_REPS}
    if backward:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(TOPOLOGY_REPS):
            topo.build_source_csr()
        e1.record()
        torch.cuda.synchronize()
        t["source_csr_and_plan_ms"] = e0.elapsed_time(e1) / TOPOLOGY_REPS
    return topo, t


def bf16_dev(torch, bits, shape, dev):
    return torch.from_numpy(bits.view(np.int16).reshape(shape)).to(dev).view(torch.bfloat16)


def roofline(bound, achieved, peak, unit, traffic=None, **extra):
    if achieved > peak:
        # an algorithmic count that the caches partly serve can exceed the peak; such a
        # count is no roofline and is never reported as one
        raise ValueError(f"algorithmic rate {achieved:.0f} {unit} above the peak {peak:.0f}")
    r = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
         "traffic": traffic}
    r.update(extra)
    return r


def record(args, name, value, ms_step, dtype, config, roof, cpu, extra):
    rec = {"metric": METRIC, "value": value, "unit": "GEdges/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": dtype, "data": "synthetic",
           "config": dict({"workload": name, "global_batch": 1, "parallelism": "single GPU"}, **config),
           "roofline": roof, "cpu_baseline": cpu}
    rec.update(extra)
    return rec


# --------------------------------------------------------------------------- workloads


def bench_dot_forward(args, g, torch, synth, ident):
    w = synth.WORKLOADS[ident]
    n, heads, c = w.n, w.heads, w.head_dim
    dev = torch.device("cuda:0")
    src, dst = synth.workload_graph(ident)
    e = int(src.size)
    log(f"workload {w.name}: n={n} e={e} H={heads} C={c} {w.dtype}")
    hosts = [synth.node_tensor(ident, i, (n, heads, c)) for i in range(3)]
    if w.dtype == "bf16":
        bits = [synth.to_bf16_bits(x) for x in hosts]
        hosts = [synth.bf16_bits_to_f32(b).reshape(n, heads, c) for b in bits]
        q, k, v = (bf16_dev(torch, b, (n, heads, c), dev) for b in bits)
        code, esz = g.GGA_BF16, 2
    else:
        q, k, v = (torch.from_numpy(x).to(dev) for x in hosts)
        code, esz = g.GGA_F32, 4
    topo, tt = per_topology(g, torch, n, torch.from_numpy(src).to(dev), torch.from_numpy(dst).to(dev))
    desc = g.make_desc(n, e, heads, c, g.GGA_SCORE_DOT, code, 1.0 / np.sqrt(c))
    out = torch.empty(n, heads, c, dtype=torch.float32, device=dev)
    lse = torch.empty(n, heads, dtype=torch.float32, device=dev)
    ws = torch.empty(max(g.lib.gga_local_attn_fwd_workspace(g.ctypes.byref(desc)), 1), dtype=torch.uint8, device=dev)

    def step(tm):
        _mark(tm, "f0")
        g.gga_local_attn_fwd(desc, q, k, v, topo.row_ptr, topo.col, topo.plan, out=out, lse=lse, ws=ws)
        _mark(tm, "f1")

    tm = Timer(torch, torch.cuda.current_stream())
    ms = tm.run(step, args.steps, args.warmup)
    kms = tm.phase_ms("f0", "f1")
    # the same step captured once in a HIP graph and replayed (launch overhead amortised)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(None)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(None)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    alg = fwd_bytes(n, e, heads, c, esz)
    ach = alg / (kms * 1e-3) / 1e9
    log(f"fwd: {ms:.3f} ms/step (launch avg {kms:.3f} ms, graph replay {graph_ms:.4f} ms), "
        f"{ach:.0f} GB/s algorithmic; {tt}")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        h64 = [x.astype(np.float64) for x in hosts]
        og = oracle.Graph(n, src, dst)
        t1 = time.perf_counter()
        oracle.local_fwd_dot(h64[0], h64[1], h64[2], og, 1.0 / np.sqrt(c))
        dt = time.perf_counter() - t1
        cores = oracle.threads()
        cpu = {"value": e / dt / 1e9, "unit": "GEdges/s", "cores": cores, "kind": "oracle",
               "sample": f"the whole forward of this workload ({e} edges, all {n} rows), fp64, {dt:.1f} s",
               "model": cpu_model()}
        # one thread on every 16th target row
        rows = np.arange(0, n, 16, dtype=np.int32)
        e1 = int((og.row_ptr[rows + 1] - og.row_ptr[rows]).sum())
        oracle.set_threads(1)
        t1 = time.perf_counter()
        oracle.local_fwd_dot(h64[0], h64[1], h64[2], og, 1.0 / np.sqrt(c), rows=rows)
        dt1 = time.perf_counter() - t1
        oracle.set_threads(cores)
        cpu["one_thread"] = {"value": e1 / dt1 / 1e9, "unit": "GEdges/s", "cores": 1,
                             "sample": f"every 16th target row ({rows.size} rows, {e1} edges), {dt1:.1f} s"}
        log(f"cpu oracle: {dt:.2f} s with {cores} threads; one thread {e1 / dt1 / 1e9:.5f} GEdges/s")
    cold = mall_cold_ms(torch, lambda: step(None), max(5, min(args.steps, 20)), dev)
    log(f"launch with the MALL flushed before each (median of {len(cold)}): {float(np.median(cold)):.3f} ms")
    traffic = counted_traffic("fwd_w3") if ident == 3 else None
    roof = roofline("hbm", ach, HBM_PEAK_GBS, "GB/s", traffic, kernel="local_fwd_kernel (+ heavy-row merge launch)",
                    alg_bytes_per_launch=alg, launch_ms=kms)
    cfg = {"nodes": n, "edges": e, "heads": heads, "head_dim": c, "storage": f"{w.dtype} q/k/v, fp32 out/lse",
           "seq_len": n}
    return record(args, w.name, e / (ms * 1e-3) / 1e9, ms, w.dtype, cfg, roof, cpu,
                  dict(tt, gedge_heads_per_s=e * heads / (ms * 1e-3) / 1e9, hbm_gbs_algorithmic=ach,
                       graph_replay_ms_per_step=graph_ms, launch_ms_median=tm.phase_median_ms("f0", "f1"),
                       launch_ms_mall_flushed_median=float(np.median(cold))))


def bench_heavy_tail(args, g, torch, synth):
    ident = 5
    w = synth.WORKLOADS[ident]
    n, heads, c = w.n, w.heads, w.head_dim
    dev = torch.device("cuda:0")
    src, dst = synth.workload_graph(ident)
    e = int(src.size)
    log(f"workload {w.name}: n={n} e={e}")
    bits = [synth.to_bf16_bits(synth.node_tensor(ident, i, (n, heads, c))) for i in range(3)]
    q, k, v = (bf16_dev(torch, b, (n, heads, c), dev) for b in bits)
    d_out_h = synth.node_tensor(ident, 0, (n, heads, c), stream=synth.GRADS)
    d_out = torch.from_numpy(d_out_h).to(dev)
    topo, tt = per_topology(g, torch, n, torch.from_numpy(src).to(dev), torch.from_numpy(dst).to(dev), True)
    desc = g.make_desc(n, e, heads, c, g.GGA_SCORE_DOT, g.GGA_BF16, 1.0 / np.sqrt(c))
    out = torch.empty(n, heads, c, dtype=torch.float32, device=dev)
    lse = torch.empty(n, heads, dtype=torch.float32, device=dev)
    grads = [torch.empty(n, heads, c, dtype=torch.float32, device=dev) for _ in range(3)]
    wsf = torch.empty(max(g.lib.gga_local_attn_fwd_workspace(g.ctypes.byref(desc)), 1), dtype=torch.uint8, device=dev)
    wsb = torch.empty(g.lib.gga_local_attn_bwd_workspace(g.ctypes.byref(desc)), dtype=torch.uint8, device=dev)

    def step(tm):
        _mark(tm, "f0")
        g.gga_local_attn_fwd(desc, q, k, v, topo.row_ptr, topo.col, topo.plan, out=out, lse=lse, ws=wsf)
        _mark(tm, "f1")
        g.gga_local_attn_bwd(desc, q, k, v, out, lse, d_out, topo, d_qs=grads[0], d_ks=grads[1], d_v=grads[2],
                             ws=wsb)
        _mark(tm, "b1")

    tm = Timer(torch, torch.cuda.current_stream())
    ms = tm.run(step, args.steps, args.warmup)
    fms, bms = tm.phase_ms("f0", "f1"), tm.phase_ms("f1", "b1")
    fa, ba = fwd_bytes(n, e, heads, c, 2), bwd_bytes(n, e, heads, c, 2)
    log(f"step {ms:.3f} ms: fwd {fms:.3f} ms ({fa / fms / 1e6:.0f} GB/s), bwd {bms:.3f} ms "
        f"({ba / bms / 1e6:.0f} GB/s); {tt}")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        h64 = [synth.bf16_bits_to_f32(b).reshape(n, heads, c).astype(np.float64) for b in bits]
        og = oracle.Graph(n, src, dst)
        t1 = time.perf_counter()
        oracle.local_fwd_dot(h64[0], h64[1], h64[2], og, 1.0 / np.sqrt(c))
        oracle.local_bwd_dot(h64[0], h64[1], h64[2], d_out_h, og, 1.0 / np.sqrt(c))
        dt = time.perf_counter() - t1
        cpu = {"value": e / dt / 1e9, "unit": "GEdges/s", "cores": oracle.threads(), "kind": "oracle",
               "sample": f"the whole step (forward + backward, {e} edges), fp64, {dt:.1f} s"}
        log(f"cpu oracle: {dt:.2f} s")
    # The roofline is the forward launch's (the metric's kernel; its per-edge count is what
    # HBM delivers: counted ~ algorithmic).  The backward call is reported beside it with its
    # counted traffic: pass B's algorithmic count charges a target row per out-edge, and the
    # caches serve much of that for hub targets, so only the counted rate is a fraction of peak.
    bwd_counted = counted_traffic("bwd_w5")
    roof = roofline("hbm", fa / (fms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", counted_traffic("fwd_w5"),
                    kernel="local_fwd_kernel (+ heavy-row merge launch)", alg_bytes_per_launch=fa, launch_ms=fms,
                    backward={"kernel": "bwd_dst_kernel + bwd_src_kernel (+ merges), one call", "ms": bms,
                              "alg_bytes": ba, "counted_gb": bwd_counted,
                              "counted_frac": bwd_counted / (bms * 1e-3) / HBM_PEAK_GBS if bwd_counted else None})
    cfg = {"nodes": n, "edges": e, "heads": heads, "head_dim": c, "storage": "bf16 q/k/v, fp32 grads",
           "step": "forward + backward", "seq_len": n}
    return record(args, w.name, e / (ms * 1e-3) / 1e9, ms, "bf16", cfg, roof, cpu,
                  dict(tt, fwd_ms=fms, bwd_ms=bms, fwd_gbs_algorithmic=fa / fms / 1e6,
                       bwd_gbs_algorithmic=ba / bms / 1e6))


def bench_edge_values(g, torch, topo, n, e, width, dev, reps=20):
    """The endpoint projection primitive at this graph's shape, timed alone: out[e] =
    x[src[e]] over an [n, width] fp32 table, and its backward dx[u] = the sum of d_edge over
    the out-edges of u, walked through the CSR by source.  The rates count each byte that
    has to move once: the table (or dx), the endpoints (or eid and row_ptr) and the
    [e, width] field."""
    x = torch.randn(n, width, device=dev)
    d_edge = torch.randn(e, width, device=dev)
    out = torch.empty(e, width, device=dev)
    dx = torch.empty(n, width, device=dev)

    def timed(f):
        f()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            f()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    fms = timed(lambda: g.gga_edge_values(x, topo.src, out=out))
    bms = timed(lambda: g.gga_edge_values_bwd(n, d_edge, topo.row_ptr_s, topo.eid_s, dx=dx))
    fb = 4 * n * width + 4 * e + 4 * e * width
    bb = 4 * (n + 1) + 4 * e + 4 * e * width + 4 * n * width
    log(f"edge_values [{e}, {width}] fp32: fwd {fms * 1e3:.1f} us ({fb / fms / 1e6:.0f} GB/s), "
        f"bwd {bms * 1e3:.1f} us ({bb / bms / 1e6:.0f} GB/s)")
    return {"width": width, "dtype": "f32", "reps": reps, "fwd_ms": fms, "fwd_bytes": fb,
            "fwd_gbs": fb / fms / 1e6, "bwd_ms": bms, "bwd_bytes": bb, "bwd_gbs": bb / bms / 1e6}


def bench_gat(args, g, torch, synth, ident):
    """The GAT layer, forward + first-order gradients; the edge-feature workload adds 16
    learned features per edge to every logit and averages the heads."""
    from sparse_graph_attention_amd import layers

    w = synth.WORKLOADS[ident]
    n, heads, c = w.n, w.heads, w.head_dim
    dev = torch.device("cuda:0")
    src, dst = synth.workload_graph(ident)
    e = int(src.size)
    log(f"workload {w.name}: n={n} e={e}")
    x, wt, a_s, a_t, d_out = synth.gat_inputs(n)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    concat, edge, edge_d = True, None, None
    if ident == 7:
        concat = False
        edge = synth.gat_edge_inputs(e)
        edge_d = {k: t(v) for k, v in edge.items()}
        d_out = synth.node_tensor(ident, 0, (n, c), stream=synth.GRADS)
    xd, wd, asd, atd, dod = t(x), t(wt), t(a_s), t(a_t), t(d_out)
    topo, tt = per_topology(g, torch, n, t(src), t(dst), True)

    def step(tm):
        _mark(tm, "f0")
        f = layers.gat_forward(xd, wd, asd, atd, topo, concat=concat, edge=edge_d)
        _mark(tm, "f1")
        layers.gat_backward(xd, wd, asd, atd, dod, f, topo, concat=concat, edge=edge_d)
        _mark(tm, "b1")

    tm = Timer(torch, torch.cuda.current_stream())
    ms = tm.run(step, args.steps, args.warmup)
    fms, bms = tm.phase_ms("f0", "f1"), tm.phase_ms("f1", "b1")
    log(f"step {ms:.3f} ms: fwd {fms:.3f} ms, bwd {bms:.3f} ms; {tt}")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        og = oracle.Graph(n, src, dst)
        t1 = time.perf_counter()
        oracle.gat_forward(x, wt, a_s, a_t, og, concat=concat, edge=edge)
        oracle.gat_backward(x, wt, a_s, a_t, d_out, og, concat=concat, edge=edge)
        dt = time.perf_counter() - t1
        cpu = {"value": e / dt / 1e9, "unit": "GEdges/s", "cores": oracle.threads(), "kind": "oracle",
               "sample": f"the whole step (layer forward + first-order gradients), fp64, {dt:.1f} s"}
    fa = fwd_bytes(n, e, heads, c, 4) + n * heads * 8 * 2  # + s_src, s_dst per edge side
    if edge is not None:
        fe = edge["f"].shape[1]
        # per edge: its feature row read, s_edge = F G written, permuted to CSR order (read +
        # write) and read by the attention kernel
        fa += e * (4 * fe + 4 * 4 * heads)
    roof = roofline("hbm", fa / (fms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", None,
                    kernel="layer forward (GEMMs, coefficients, fused local forward)", alg_bytes_per_launch=fa,
                    launch_ms=fms)
    cfg = {"nodes": n, "edges": e, "heads": heads, "head_dim": c, "fin": w.fin, "storage": "fp32",
           "heads_combined": "concatenated" if concat else "averaged",
           "edge_features": 0 if edge is None else int(edge["f"].shape[1]),
           "step": "forward + first-order gradients", "seq_len": n}
    extra = dict(tt, fwd_ms=fms, bwd_ms=bms)
    if ident == 2:
        extra["edge_values"] = bench_edge_values(g, torch, topo, n, e, heads, dev)
    return record(args, w.name, e / (ms * 1e-3) / 1e9, ms, "f32", cfg, roof, cpu, extra)


def bench_layer(args, g, torch, synth, ident):
    """The gated local-global layer, forward + gradients of every input and parameter; for a
    batched workload the graphs are packed along the node axis (block-diagonal edges,
    per-graph global statistics)."""
    from sparse_graph_attention_amd import layers

    w = synth.WORKLOADS[ident]
    n, heads, c, d = w.n, w.heads, w.head_dim, w.d_model
    dev = torch.device("cuda:0")
    node_ptr = node_ptr_d = None
    if w.batch > 1:
        node_ptr, edge_ptr, sl, dl = synth.workload_batch(ident)
        node_ptr_d = torch.from_numpy(node_ptr).to(dev)
        src_d, dst_d, bad = g.gga_batch_edges(node_ptr_d, torch.from_numpy(edge_ptr).to(dev),
                                              torch.from_numpy(sl).to(dev), torch.from_numpy(dl).to(dev))
        torch.cuda.synchronize()
        if int(bad.item()) != 0:
            raise RuntimeError("batch packing found ids outside their graph")
    else:
        src, dst = synth.workload_graph(ident)
        src_d, dst_d = torch.from_numpy(src).to(dev), torch.from_numpy(dst).to(dev)
    e = int(src_d.numel())
    log(f"workload {w.name}: n={n} e={e} graphs={w.batch}")
    p = synth.gated_layer_inputs(n, d=d, ident=ident)
    d_out = synth.node_tensor(ident, 7, (n, d))
    pd = {k: (torch.from_numpy(np.ascontiguousarray(v)).to(dev) if isinstance(v, np.ndarray) else v)
          for k, v in p.items()}
    dod = torch.from_numpy(d_out).to(dev)
    topo, tt = per_topology(g, torch, n, src_d, dst_d, True)

    def step(tm):
        _mark(tm, "f0")
        f = layers.gated_layer_forward(pd, topo, heads, node_ptr=node_ptr_d)
        _mark(tm, "f1")
        layers.gated_layer_backward(pd, f, topo, heads, dod, node_ptr=node_ptr_d,
                                    mark=None if tm is None else (lambda name: _mark(tm, name)))
        _mark(tm, "b1")

    tm = Timer(torch, torch.cuda.current_stream())
    ms = tm.run(step, args.steps, args.warmup)
    fms, bms = tm.phase_ms("f0", "f1"), tm.phase_ms("f1", "b1")
    # dense contractions: 4 forward and 8 backward n x d x d products; the global branch's
    # per-head r x r contractions (2 forward, 5 backward)
    flops = 2.0 * n * d * d * 12 + 2.0 * n * heads * c * c * 7
    log(f"step {ms:.3f} ms: fwd {fms:.3f} ms, bwd {bms:.3f} ms ({flops / ms / 1e9:.1f} TFLOP/s over the dense "
        f"contractions); {tt}")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        if node_ptr is not None:
            src, dst, _ = oracle.batch_edges(node_ptr, edge_ptr, sl, dl)
        og = oracle.Graph(n, src, dst)
        t1 = time.perf_counter()
        oracle.gated_layer_backward(p, og, heads, d_out, node_ptr=node_ptr)
        dt = time.perf_counter() - t1
        cpu = {"value": e / dt / 1e9, "unit": "GEdges/s", "cores": oracle.threads(), "kind": "oracle",
               "sample": f"the whole step (layer forward + first-order gradients), fp64 (numpy matmuls for the "
                         f"dense products), {dt:.1f} s"}
    kms = tm.phase_ms("local_bwd0", "local_bwd1")
    if node_ptr is None:
        # the dominant call of the step: the local attention's backward (pass A over the CSR
        # by destination, pass B over the CSR by source, the merges), HBM bound
        alg = bwd_bytes(n, e, heads, c, 4)
        roof = roofline("hbm", alg / (kms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", counted_traffic("bwd_w4"),
                        kernel="local attention backward call (bwd_dst_kernel, bwd_src_kernel, bwd_merge)",
                        alg_bytes_per_launch=alg, launch_ms=kms, step_share=kms / ms,
                        dense_tflops_per_step=flops / (ms * 1e-3) / 1e12)
    else:
        # small graphs: each graph's key and value rows stay in the caches, so a per-edge byte
        # count is no HBM count; the step's dense contractions are its roofline
        roof = roofline("mfma", flops / (ms * 1e-3) / 1e12, MFMA_F32_PEAK_TFLOPS, "TFLOP/s", None,
                        kernel="whole layer step (fp32 GEMMs dominate the flops)", flops_per_step=flops,
                        launch_ms=ms, local_bwd_ms=kms)
    cfg = {"nodes": n, "edges": e, "heads": heads, "head_dim": c, "d_model": d, "graphs": w.batch,
           "storage": "fp32", "step": "layer forward + first-order gradients", "seq_len": n}
    return record(args, w.name, e / (ms * 1e-3) / 1e9, ms, "f32", cfg, roof, cpu, dict(tt, fwd_ms=fms, bwd_ms=bms))


def bench_relation(args, g, torch, synth, ident):
    """Relation-typed messages (per-relation key and message transforms of every node,
    mean or softmax weighting over each target's in-edges), forward + gradients of the
    input and every transform, over a packed batch of token sequences."""
    from sparse_graph_attention_amd import layers

    w = synth.WORKLOADS[ident]
    n, heads, c, d, n_rel = w.n, w.heads, w.head_dim, w.d_model, w.relations
    mean = w.score == "mean"
    width = heads * c
    dev = torch.device("cuda:0")
    _, src, dst, rel, segs = synth.workload_relation_edges(ident)
    e = int(src.size)
    log(f"workload {w.name}: n={n} e={e} relations={n_rel} mode={'mean' if mean else 'softmax'}")
    p = synth.relation_inputs(n, d, heads, c, n_rel, ident=8)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)  # noqa: E731
    xd, wqd = t(p["x"]), t(p["w_q"])
    wkd, wvd = t(np.concatenate(list(p["w_k"]), 1)), t(np.concatenate(list(p["w_v"]), 1))
    dod = t(p["d_out"])
    src_d, dst_d = torch.from_numpy(src).to(dev), torch.from_numpy(dst).to(dev)
    layers.relation_topology(n, n_rel, src_d, dst_d, segs, backward=True)  # untimed warm-up build
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    topo, bad = layers.relation_topology(n, n_rel, src_d, dst_d, segs, backward=True)
    e1.record()
    torch.cuda.synchronize()
    if int(bad.item()) != 0:
        raise RuntimeError("relation edges with endpoints outside the batch")
    tt = {"relation_rows_csrs_and_plans_ms": e0.elapsed_time(e1)}

    def step(tm):
        _mark(tm, "f0")
        f = layers.relation_forward(xd, wqd, wkd, wvd, topo, heads, n_rel, mean)
        _mark(tm, "f1")
        layers.relation_backward(xd, wqd, wkd, wvd, dod, f, topo, heads, n_rel, mean)
        _mark(tm, "b1")

    tm = Timer(torch, torch.cuda.current_stream())
    ms = tm.run(step, args.steps, args.warmup)
    fms, bms = tm.phase_ms("f0", "f1"), tm.phase_ms("f1", "b1")
    # the attention kernels alone, on the layer's own tensors
    f = layers.relation_forward(xd, wqd, wkd, wvd, topo, heads, n_rel, mean)
    desc = f["desc"]
    fws = torch.empty(g.lib.gga_local_attn_fwd_workspace(ctypes.byref(desc)) + 1, dtype=torch.uint8, device=dev)
    bws = torch.empty(g.lib.gga_local_attn_bwd_workspace(ctypes.byref(desc)) + 1, dtype=torch.uint8, device=dev)
    d3 = dod.view(n, heads, c)
    grads = [None, None, torch.empty_like(f["v"], dtype=torch.float32)]
    if not mean:
        grads[0], grads[1] = torch.empty_like(f["q"]), torch.empty_like(f["k"])

    def attn(tm):
        _mark(tm, "a0")
        g.gga_local_attn_fwd(desc, f["q"], f["k"], f["v"], topo.row_ptr, topo.col, topo.plan, out=f["out3"],
                             lse=f["lse"], want_lse=not mean, ws=fws)
        _mark(tm, "a1")
        g.gga_local_attn_bwd(desc, f["q"], f["k"], f["v"], f["out3"], f["lse"], d3, topo, *grads, ws=bws)
        _mark(tm, "a2")

    ta = Timer(torch, torch.cuda.current_stream())
    ta.run(attn, args.steps, args.warmup)
    afms, abms = ta.phase_ms("a0", "a1"), ta.phase_ms("a1", "a2")
    ns = n * n_rel
    if mean:
        # forward: a message row and col per edge, row_ptr, out; backward (CSR by source): per
        # edge a dO row, col and the target's two row_ptr entries; row_ptr_s; d_v written
        fa = e * (4 * width + 4) + 4 * (n + 1) + 4 * n * width
        ba = e * (4 * width + 4 + 8) + 4 * (ns + 1) + 4 * ns * width
    else:
        fa = fwd_bytes(n, e, heads, c, 4)
        ba = (e * (2 * 4 * width + 4) + n * (4 * width + 8 * width + 4 * heads + 4) + n * (4 * width + 4 * heads)
              + e * (4 * width + 4 * width + 8 * heads + 4) + ns * (2 * 4 * width + 4) + ns * 8 * width)
    # every transform's product appears three times (forward, its weight gradient, dX)
    flops = 3 * 2.0 * n * d * (n_rel * width + (0 if mean else width + n_rel * width))
    log(f"step {ms:.3f} ms: fwd {fms:.3f} ms, bwd {bms:.3f} ms ({flops / ms / 1e9:.1f} TFLOP/s over the "
        f"projections); attention alone fwd {afms:.3f} ms ({fa / afms / 1e6:.0f} GB/s), bwd {abms:.3f} ms "
        f"({ba / abms / 1e6:.0f} GB/s); {tt}")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        omode = oracle.REL_MEAN if mean else oracle.REL_SOFTMAX
        t1 = time.perf_counter()
        oracle.relation_forward(p["x"], p["w_q"], p["w_k"], p["w_v"], src, dst, rel, heads, omode)
        oracle.relation_backward(p["x"], p["w_q"], p["w_k"], p["w_v"], src, dst, rel, heads, omode, p["d_out"])
        dt = time.perf_counter() - t1
        cpu = {"value": e / dt / 1e9, "unit": "GEdges/s", "cores": oracle.threads(), "kind": "oracle",
               "sample": f"the whole step (forward + first-order gradients), fp64 (numpy matmuls for the "
                         f"projections), {dt:.1f} s"}
    roof = roofline("mfma", flops / (ms * 1e-3) / 1e12, MFMA_F32_PEAK_TFLOPS, "TFLOP/s", None,
                    kernel="whole step (fp32 projections dominate)", flops_per_step=flops, launch_ms=ms,
                    # algorithmic bytes over time: a sequence's (token, relation) rows are read only
                    # by that sequence's edges (256 tokens x 3 relations x 2 KiB each for K, the same
                    # for V), so the caches serve most of the gathers and this rate can exceed the
                    # HBM peak; it is not an HBM fraction
                    attention_fwd={"ms": afms, "alg_bytes": fa, "alg_GB_s": fa / afms / 1e6,
                                   "note": "cache-served; not bounded by the HBM peak"},
                    attention_bwd={"ms": abms, "alg_bytes": ba, "alg_GB_s": ba / abms / 1e6,
                                   "note": "cache-served; not bounded by the HBM peak"})
    cfg = {"nodes": n, "edges": e, "heads": heads, "head_dim": c, "d_model": d, "relations": n_rel,
           "weighting": "mean" if mean else "softmax", "sequences": w.batch, "seq_len": n // w.batch,
           "storage": "fp32", "step": "forward + first-order gradients"}
    return record(args, w.name, e / (ms * 1e-3) / 1e9, ms, "f32", cfg, roof, cpu, dict(tt, fwd_ms=fms, bwd_ms=bms))


def stream_rates(torch, n=262144 * 256, reps=20):
    """Best-of-reps rates of torch's own elementwise kernels on [2^18, 256] fp32 tensors (the
    gated layer's row tensors): the streaming rate a row-wise kernel of that size can reach
    here, for one, two and three reads per write, and for a copy that moves one head's
    256-byte segment of every row at a time (the access pattern of the global branch's
    per-head passes)."""
    dev = torch.device("cuda:0")
    a, b, c, d = (torch.randn(n, device=dev) for _ in range(4))
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nb = n * 4
    a4, c4 = a.view(-1, 4, 64), c.view(-1, 4, 64)

    def head_slices():  # one head's 256-byte segment of each 1 KiB row, the four heads in turn
        for h in range(4):
            c4[:, h].copy_(a4[:, h])

    for name, fn, moved in (("copy (1 read, 1 write)", lambda: c.copy_(a), 2 * nb),
                            ("add (2 reads, 1 write)", lambda: torch.add(a, b, out=c), 3 * nb),
                            ("addcmul (3 reads, 1 write)", lambda: torch.addcmul(a, b, d, out=c), 4 * nb),
                            ("copy by head slices (1 read, 1 write)", head_slices, 2 * nb)):
        for _ in range(3):
            fn()
        best = float("inf")
        for _ in range(reps):
            s.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            best = min(best, s.elapsed_time(e))
        log(f"stream rate {name}: {best * 1e3:.1f} us, {moved / best / 1e9:.2f} TB/s")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5, 6, 7, 8, 9])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--stream-rates", action="store_true",
                    help="also time plain torch elementwise kernels (copy, add, addcmul) over 268 MB "
                         "fp32 tensors: the streaming rates of read/write mixes on this device")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures a single GPU; --gpus above 1 is not supported",
              file=sys.stderr)
        return 2

    import torch

    import sparse_graph_attention_amd as g
    import synth

    if args.workload in (1, 3):
        rec = bench_dot_forward(args, g, torch, synth, args.workload)
    elif args.workload == 5:
        rec = bench_heavy_tail(args, g, torch, synth)
    elif args.workload in (2, 7):
        rec = bench_gat(args, g, torch, synth, args.workload)
    elif args.workload in (8, 9):
        rec = bench_relation(args, g, torch, synth, args.workload)
    else:
        rec = bench_layer(args, g, torch, synth, args.workload)
    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies done")
    if args.stream_rates:
        stream_rates(torch)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
