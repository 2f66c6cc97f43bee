"""GPU parity of the batched (packed multi-graph) path against the oracle ("Gated
Local-Global Graph Attention", Implementation notes note 1: a batch of graphs, one adjacency
list each): the block-diagonal packing (bit-exact), the per-graph global branch forward and
backward over batches of very different graph sizes (empty graphs, graphs of one node,
hundreds of short graphs in one tile, long graphs cut over many tiles), and the batched
layer forward + backward, including the 64-graph workload."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, global_term_scales, i32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import sparse_graph_attention_amd as m

    return m


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def _ptr(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


BATCHES = {
    "ragged": (1, 0, 17, 300, 4096, 2, 1000, 0, 2500, 63),
    "tiny": tuple((np.arange(700) % 5 + 1).tolist()),  # 700 graphs of 1-5 nodes
    "long": (5000, 3, 7000, 256, 257, 512),  # tile-boundary sizes for 256-row tiles
    # 104,779 rows: tiles longer than 256 rows (416 at 4 heads, 320 at 3), graphs longer than
    # one tile starting inside tiles
    "long_tiles": (40000, 593, 1, 30000, 1185, 0, 33000),
    "one": (3000,),
    "empty_tail": (40, 0, 0),
}


def test_batch_edges_bit_exact(g):
    node_ptr, edge_ptr, sl, dl = synth.ragged_batch(1)
    sl = sl.copy()
    dl = dl.copy()
    # plant ids outside their graph: too large, negative, and one graph's entries shifted
    sl[5] = 10_000
    dl[9] = -2
    sl[edge_ptr[3]:edge_ptr[3] + 4] += int(node_ptr[4] - node_ptr[3])
    src, dst, bad = oracle.batch_edges(node_ptr, edge_ptr, sl, dl)
    s_d, d_d, b_d = g.gga_batch_edges(i32(node_ptr), i32(edge_ptr), i32(sl), i32(dl))
    torch.cuda.synchronize()
    assert np.array_equal(s_d.cpu().numpy(), src)
    assert np.array_equal(d_d.cpu().numpy(), dst)
    assert int(b_d.item()) == bad and bad >= 3


def test_batch_edges_then_csr(g):
    """The packed list goes straight into the CSR build; bit-exact against the oracle's CSR."""
    node_ptr, edge_ptr, sl, dl = synth.ragged_batch(2)
    src, dst, _ = oracle.batch_edges(node_ptr, edge_ptr, sl, dl)
    s_d, d_d, b_d = g.gga_batch_edges(i32(node_ptr), i32(edge_ptr), i32(sl), i32(dl))
    n = int(node_ptr[-1])
    row_ptr, col, eid = g.gga_coo_to_csr(n, d_d, s_d)
    torch.cuda.synchronize()
    assert int(b_d.item()) == 0
    o_rp, o_col, o_eid = oracle.coo_to_csr(n, dst, src)
    assert np.array_equal(row_ptr.cpu().numpy(), o_rp)
    assert np.array_equal(col.cpu().numpy(), o_col)
    assert np.array_equal(eid.cpu().numpy(), o_eid)


@pytest.mark.parametrize("name", sorted(BATCHES))
@pytest.mark.parametrize("heads,r", [(4, 64), (2, 16), (3, 24)])
def test_global_batch_fwd(g, name, heads, r):
    sizes = BATCHES[name]
    node_ptr = _ptr(sizes)
    n = int(node_ptr[-1])
    print(f"global batch fwd {name}: n={n} graphs={len(sizes)} H={heads} r={r}", flush=True)
    q, k, v = (_rand((n, heads, r), 60 + i) for i in range(3))
    s, z, gg = g.gga_global_linear_batch_fwd(i32(node_ptr), _t(q), _t(k), _t(v), 1e-6)
    torch.cuda.synchronize()
    rs, rz, rg = oracle.global_linear_seg(q, k, v, node_ptr, 1e-6)
    biggest = max(max(sizes), 1)
    assert_close(s.cpu().numpy(), rs, "f32", "S", atol=1e-5 * np.sqrt(biggest))
    assert_close(z.cpu().numpy(), rz, "f32", "z", atol=1e-5 * np.sqrt(biggest))
    assert_close(gg.cpu().numpy(), rg, "f32", "G")


@pytest.mark.parametrize("name", sorted(BATCHES))
@pytest.mark.parametrize("heads,r", [(4, 64), (3, 24)])
def test_global_batch_bwd(g, name, heads, r):
    sizes = BATCHES[name]
    node_ptr = _ptr(sizes)
    n = int(node_ptr[-1])
    print(f"global batch bwd {name}: n={n} graphs={len(sizes)} H={heads} r={r}", flush=True)
    q, k, v, d_g = (_rand((n, heads, r), 70 + i) for i in range(4))
    ref = oracle.global_linear_seg_bwd(q, k, v, d_g, node_ptr, 1e-6)
    scale = global_term_scales(q, k, v, d_g, 1e-6, node_ptr=node_ptr)
    names = ("d_q", "d_k", "d_v")
    np_d = i32(node_ptr)
    qd, kd, vd, gd = _t(q), _t(k), _t(v), _t(d_g)
    s, z, gfw = g.gga_global_linear_batch_fwd(np_d, qd, kd, vd, 1e-6)
    grads = [torch.zeros(n, heads, r, device="cuda") for _ in names]
    g.gga_global_linear_batch_bwd(np_d, qd, kd, vd, s, z, gd, *grads, 1e-6)
    # with the forward's G the query pass reads dG . G instead of forming num again
    grads_g = [torch.zeros(n, heads, r, device="cuda") for _ in names]
    g.gga_global_linear_batch_bwd(np_d, qd, kd, vd, s, z, gd, *grads_g, 1e-6, g_fw=gfw)
    # the kernels add into what is there: from a nonzero start the result is that start plus
    # the same contribution (the addition may be fused with the last product, so the two
    # differ by at most a rounding of each)
    base = [_t(_rand((n, heads, r), 80 + i)) for i in range(3)]
    acc = [b.clone() for b in base]
    g.gga_global_linear_batch_bwd(np_d, qd, kd, vd, s, z, gd, *acc, 1e-6)
    torch.cuda.synchronize()
    for got, nm in zip(grads_g, names):
        assert_close(got.cpu().numpy(), ref[nm], "f32", nm + " (forward G)", atol=1e-5 * scale[nm])
    for got, b, a, nm in zip(grads, base, acc, names):
        assert_close(got.cpu().numpy(), ref[nm], "f32", nm, atol=1e-5 * scale[nm])
        lim = 2.0 ** -23 * (b.abs() + 2 * got.abs())
        assert bool(((a - (b + got)).abs() <= lim).all()), nm


def test_global_batch_of_one_equals_plain(g):
    """A batch holding one graph runs the same kernels as the plain entry point: identical
    bits."""
    n, heads, r = 5000, 4, 64
    q, k, v, d_g = (_t(_rand((n, heads, r), 90 + i)) for i in range(4))
    np_d = i32(np.array([0, n], np.int32))
    s1, z1, g1 = g.gga_global_linear_fwd(q, k, v, 1e-6)
    s2, z2, g2 = g.gga_global_linear_batch_fwd(np_d, q, k, v, 1e-6)
    a = [torch.zeros(n, heads, r, device="cuda") for _ in range(3)]
    b = [torch.zeros(n, heads, r, device="cuda") for _ in range(3)]
    g.gga_global_linear_bwd(q, k, v, s1, z1, d_g, *a, 1e-6)
    g.gga_global_linear_batch_bwd(np_d, q, k, v, s2, z2, d_g, *b, 1e-6)
    ag = [torch.zeros(n, heads, r, device="cuda") for _ in range(3)]
    bg = [torch.zeros(n, heads, r, device="cuda") for _ in range(3)]
    g.gga_global_linear_bwd(q, k, v, s1, z1, d_g, *ag, 1e-6, g_fw=g1)
    g.gga_global_linear_batch_bwd(np_d, q, k, v, s2, z2, d_g, *bg, 1e-6, g_fw=g2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2[0]) and torch.equal(z1, z2[0]) and torch.equal(g1, g2)
    for x, y in zip(a + ag, b + bg):
        assert torch.equal(x, y)


def _dev(p):
    return {kk: (torch.from_numpy(np.ascontiguousarray(vv)).cuda() if isinstance(vv, np.ndarray) else vv)
            for kk, vv in p.items()}


def _close(got, want, what):
    got = got.cpu().numpy() if isinstance(got, torch.Tensor) else got
    want = np.asarray(want, np.float64)
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    return assert_close(got, want, "f32", what, atol=1e-5 * rms + 1e-30)


def _batched_layer(g, node_ptr, edge_ptr, sl, dl, heads, p, d_out):
    from sparse_graph_attention_amd import layers

    n = int(node_ptr[-1])
    np_d = i32(node_ptr)
    s_d, d_d, bad = g.gga_batch_edges(np_d, i32(edge_ptr), i32(sl), i32(dl))
    topo = g.Topology(n, s_d, d_d, backward=True)
    pd = _dev(p)
    fwd = layers.gated_layer_forward(pd, topo, heads, node_ptr=np_d)
    grads = layers.gated_layer_backward(pd, fwd, topo, heads, _t(d_out), node_ptr=np_d)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    src, dst, _ = oracle.batch_edges(node_ptr, edge_ptr, sl, dl)
    ref = oracle.gated_layer_backward(p, oracle.Graph(n, src, dst), heads, d_out, node_ptr=node_ptr)
    f = ref["fwd"]
    _close(fwd["out"], f["out"], "out")
    _close(fwd["glob"], f["glob"], "glob")
    for name in ("d_x", "d_w_q", "d_w_k", "d_w_v", "d_w_o", "d_w_g", "d_gamma", "d_beta"):
        _close(grads[name], ref[name], name)
    _close(grads["d_b_g"], np.array([ref["d_b_g"]]), "d_b_g")


def test_batched_layer_ragged(g):
    node_ptr, edge_ptr, sl, dl = synth.ragged_batch(3)
    n = int(node_ptr[-1])
    p = synth.gated_layer_inputs(n, d=256)
    _batched_layer(g, node_ptr, edge_ptr, sl, dl, 4, p, _rand((n, 256), 95))


def test_batched_layer_workload(g):
    w = synth.WORKLOADS[6]
    node_ptr, edge_ptr, sl, dl = synth.workload_batch(6)
    print(f"workload {w.name}: n={w.n} graphs={w.batch} e={sl.size}", flush=True)
    p = synth.gated_layer_inputs(w.n, d=w.d_model, ident=6)
    _batched_layer(g, node_ptr, edge_ptr, sl, dl, w.heads, p, _rand((w.n, w.d_model), 96))
