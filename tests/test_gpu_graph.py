"""HIP graph capture of the library's calls.

Every entry point only enqueues kernels (no allocation, no memset node, no host sync), so
a caller can capture a whole step -- CSR build, plan, forward, backward -- in a HIP graph
and replay it.  Each replay is checked against the eager result, with eager work and
synchronisations between replays."""

import numpy as np
import pytest
import torch

import synth
from gpu_util import i32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import sparse_graph_attention_amd as m

    return m


def test_graph_capture_and_replay(g):
    n = 3000
    src, dst = synth.mixed_degree_graph(n, 41, hubs=(5000, 1500, 300))
    e = src.size
    rng = np.random.default_rng(7)
    heads, c = 8, 32
    q, k, v = (torch.from_numpy(rng.standard_normal((n, heads, c)).astype(np.float32)).cuda().bfloat16()
               for _ in range(3))
    d_out = torch.from_numpy(rng.standard_normal((n, heads, c)).astype(np.float32)).cuda()
    src_d, dst_d = i32(src), i32(dst)
    desc = g.make_desc(n, e, heads, c, g.GGA_SCORE_DOT, g.GGA_BF16)

    # every buffer the step touches is allocated up front
    def bufs():
        b = dict(row_ptr=torch.empty(n + 1, dtype=torch.int32, device="cuda"),
                 col=torch.empty(e, dtype=torch.int32, device="cuda"),
                 eid=torch.empty(e, dtype=torch.int32, device="cuda"),
                 row_ptr_s=torch.empty(n + 1, dtype=torch.int32, device="cuda"),
                 col_s=torch.empty(e, dtype=torch.int32, device="cuda"),
                 eid_s=torch.empty(e, dtype=torch.int32, device="cuda"),
                 plan=torch.empty(g.lib.gga_plan_bytes(n, e), dtype=torch.uint8, device="cuda"),
                 plan_s=torch.empty(g.lib.gga_plan_bytes(n, e), dtype=torch.uint8, device="cuda"),
                 ws_csr=torch.empty(g.lib.gga_coo_to_csr_workspace(n, e), dtype=torch.uint8, device="cuda"),
                 ws_plan=torch.empty(g.lib.gga_plan_workspace(n, e), dtype=torch.uint8, device="cuda"),
                 ws_f=torch.empty(g.lib.gga_local_attn_fwd_workspace(g.ctypes.byref(desc)), dtype=torch.uint8,
                                  device="cuda"),
                 ws_b=torch.empty(g.lib.gga_local_attn_bwd_workspace(g.ctypes.byref(desc)), dtype=torch.uint8,
                                  device="cuda"),
                 out=torch.empty(n, heads, c, device="cuda"), lse=torch.empty(n, heads, device="cuda"),
                 dq=torch.empty(n, heads, c, device="cuda"), dk=torch.empty(n, heads, c, device="cuda"),
                 dv=torch.empty(n, heads, c, device="cuda"))
        return b

    def step(b):
        g.gga_coo_to_csr(n, dst_d, src_d, b["row_ptr"], b["col"], b["eid"], ws=b["ws_csr"])
        g.gga_plan_build(n, e, b["row_ptr"], plan=b["plan"], ws=b["ws_plan"])
        g.gga_coo_to_csr(n, src_d, dst_d, b["row_ptr_s"], b["col_s"], b["eid_s"], ws=b["ws_csr"])
        g.gga_plan_build(n, e, b["row_ptr_s"], plan=b["plan_s"], ws=b["ws_plan"])
        g.gga_local_attn_fwd(desc, q, k, v, b["row_ptr"], b["col"], b["plan"], out=b["out"], lse=b["lse"],
                             ws=b["ws_f"])
        topo = g.Topology.__new__(g.Topology)
        topo.row_ptr, topo.col, topo.plan = b["row_ptr"], b["col"], b["plan"]
        topo.row_ptr_s, topo.col_s, topo.plan_s = b["row_ptr_s"], b["col_s"], b["plan_s"]
        g.gga_local_attn_bwd(desc, q, k, v, b["out"], b["lse"], d_out, topo, d_qs=b["dq"], d_ks=b["dk"],
                             d_v=b["dv"], ws=b["ws_b"])

    eager = bufs()
    step(eager)
    torch.cuda.synchronize()

    cap = bufs()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(cap)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(cap)
    for rep in range(4):
        for t in cap.values():  # scribble over every output so a replay must rewrite it
            if t.dtype == torch.float32:
                t.fill_(float("nan"))
            elif t.dtype == torch.int32:
                t.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        x = torch.randn(1000, 1000, device="cuda") @ torch.randn(1000, 1000, device="cuda")  # eager work between
        torch.cuda.synchronize()
        for name in ("row_ptr", "col", "eid", "row_ptr_s", "col_s", "eid_s", "out", "lse", "dq", "dk", "dv"):
            assert torch.equal(cap[name], eager[name]), (rep, name)
        del x
