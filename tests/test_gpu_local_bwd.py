"""GPU parity of the local attention backward (pass A over the CSR by destination, the
CSR-by-source transpose, pass B over it) against the oracle's closed-form gradients.

The GPU backward consumes the GPU forward's out and lse, as a caller would; the oracle
recomputes everything in fp64 from the same inputs.  Graphs have long rows in both
orientations so that the chunked-and-merged paths of both passes run."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, i32, node_pair

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import sparse_graph_attention_amd as m

    return m


def _bwd(g, n, src, dst, heads, c, dtype, score, seed, rows_d=None, rows_s=None, tensors=None):
    print(f"bwd n={n} e={src.size} H={heads} C={c} {dtype} {'dot' if score == 0 else 'add'}", flush=True)
    rng = np.random.default_rng(seed)
    og = oracle.Graph(n, src, dst)
    topo = g.Topology(n, i32(src), i32(dst), backward=True)
    scale = c ** -0.5
    if tensors is None:
        vh, vd = node_pair(rng.standard_normal((n, heads, c)).astype(np.float32), dtype)
        d_out = rng.standard_normal((n, heads, c)).astype(np.float32)
        if score == g.GGA_SCORE_DOT:
            qh, qd = node_pair(rng.standard_normal((n, heads, c)).astype(np.float32), dtype)
            kh, kd = node_pair(rng.standard_normal((n, heads, c)).astype(np.float32), dtype)
        else:
            qh = rng.standard_normal((n, heads)).astype(np.float32)
            kh = rng.standard_normal((n, heads)).astype(np.float32)
            qd, kd = torch.from_numpy(qh).cuda(), torch.from_numpy(kh).cuda()
    else:
        qh, qd, kh, kd, vh, vd, d_out = tensors
    code = g.GGA_BF16 if dtype == "bf16" else g.GGA_F32
    desc = g.make_desc(n, src.size, heads, c, score, code, scale)
    out, lse = g.gga_local_attn_fwd(desc, qd, kd, vd, topo.row_ptr, topo.col, topo.plan)
    d_out_d = torch.from_numpy(d_out).cuda()
    dq, dk, dv = g.gga_local_attn_bwd(desc, qd, kd, vd, out, lse, d_out_d, topo)
    torch.cuda.synchronize()
    if score == g.GGA_SCORE_DOT:
        r = oracle.local_bwd_dot(qh, kh, vh, d_out, og, scale, rows_d=rows_d, rows_s=rows_s)
        ref_q, ref_k, ref_v = r["d_q"], r["d_k"], r["d_v"]
    else:
        r = oracle.local_bwd_add(kh, qh, vh, d_out, og, 0.2, rows_d=rows_d, rows_s=rows_s)
        ref_q, ref_k, ref_v = r["d_s_dst"], r["d_s_src"], r["d_hf"]
    dq, dk, dv = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    if rows_d is not None:
        dq = dq[rows_d]
    if rows_s is not None:
        dk, dv = dk[rows_s], dv[rows_s]
    assert_close(dq, ref_q, dtype, "d_q")
    assert_close(dk, ref_k, dtype, "d_k")
    assert_close(dv, ref_v, dtype, "d_v")


SHAPES = [
    (1, 16, "f32", 0), (8, 64, "bf16", 0), (8, 32, "bf16", 0), (4, 64, "f32", 0), (8, 8, "f32", 1),
    (1, 1, "f32", 1), (2, 3, "f32", 0), (3, 5, "bf16", 0), (16, 64, "bf16", 0), (12, 32, "f32", 0),
    (8, 16, "bf16", 1), (2, 6, "f32", 1),
    # the widest layouts: 32 and 64 lanes per head, two full fp32 slots, additive with two slots
    (2, 256, "bf16", 0), (1, 256, "f32", 0), (1, 512, "bf16", 0), (8, 64, "f32", 0), (16, 32, "f32", 1),
    (64, 1, "f32", 0),
]


@pytest.mark.parametrize("heads,c,dtype,score", SHAPES)
def test_bwd_shapes_small(g, heads, c, dtype, score):
    src, dst = synth.random_multigraph(300, 2500, 8, isolated=5)
    _bwd(g, 300, src, dst, heads, c, dtype, score, seed=11)


@pytest.mark.parametrize("transpose", [False, True])
@pytest.mark.parametrize("heads,c,dtype,score", [(8, 32, "bf16", 0), (8, 8, "f32", 1), (2, 3, "f32", 0),
                                                 (16, 64, "bf16", 0)])
def test_bwd_all_buckets(g, heads, c, dtype, score, transpose):
    n = 4000
    src, dst = synth.mixed_degree_graph(n, 6, hubs=(9000, 3000, 1025, 1024, 700, 65, 64))
    if transpose:  # long rows in the CSR by source instead
        src, dst = dst, src
    _bwd(g, n, src, dst, heads, c, dtype, score, seed=12)


def test_bwd_edge_cases(g):
    _bwd(g, 1, np.array([0], np.int32), np.array([0], np.int32), 2, 8, "f32", 0, seed=13)
    _bwd(g, 6, np.zeros(0, np.int32), np.zeros(0, np.int32), 2, 8, "f32", 0, seed=14)
    _bwd(g, 3, np.array([1, 1, 1, 2], np.int32), np.array([0, 0, 0, 0], np.int32), 1, 4, "f32", 1, seed=15)


def test_bwd_deterministic(g):
    n = 3000
    src, dst = synth.mixed_degree_graph(n, 7, hubs=(5000, 2000))
    topo = g.Topology(n, i32(src), i32(dst), backward=True)
    rng = np.random.default_rng(1)
    q, k, v = (torch.from_numpy(rng.standard_normal((n, 8, 32)).astype(np.float32)).cuda().bfloat16()
               for _ in range(3))
    d_out = torch.from_numpy(rng.standard_normal((n, 8, 32)).astype(np.float32)).cuda()
    desc = g.make_desc(n, src.size, 8, 32, 0, g.GGA_BF16)
    out, lse = g.gga_local_attn_fwd(desc, q, k, v, topo.row_ptr, topo.col, topo.plan)
    a = g.gga_local_attn_bwd(desc, q, k, v, out, lse, d_out, topo)
    b = g.gga_local_attn_bwd(desc, q, k, v, out, lse, d_out, topo)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_workload_heavy_tail_bwd_full(g):
    """The heavy-tailed 2M-node workload: forward, then dQ over the CSR by destination and
    dK, dV over the CSR by source; every row compared."""
    ident = 5
    w = synth.WORKLOADS[ident]
    n, heads, c = w.n, w.heads, w.head_dim
    src, dst = synth.workload_graph(ident)
    print(f"workload {w.name}: n={n} e={src.size}", flush=True)
    qh, qd = node_pair(synth.node_tensor(ident, 0, (n, heads, c)), "bf16")
    kh, kd = node_pair(synth.node_tensor(ident, 1, (n, heads, c)), "bf16")
    vh, vd = node_pair(synth.node_tensor(ident, 2, (n, heads, c)), "bf16")
    d_out = synth.node_tensor(ident, 0, (n, heads, c), stream=synth.GRADS)
    _bwd(g, n, src, dst, heads, c, "bf16", 0, seed=0, tensors=(qh, qd, kh, kd, vh, vd, d_out))
