"""GPU parity of the GAT variants the Tinymesh page lists as not yet covered (section
"Evidence and limits"), read as in the GATConv its "Reference contract" follows: learned
edge features in the score and head averaging.  The edge-term attention alone over every
degree bucket and lane layout, head averaging, and the layer forward + first-order
gradients (small graphs and the 170k-node power-law workload) against the oracle.

LeakyReLU has a kink at z = 0 where fp32 and fp64 may take different one-sided
derivatives; these tests move every edge logit at least 1e-4 away from it by construction
(the edge term, or an edge's feature row, is nudged), so every element is held to the
standard tolerance."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, i32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import sparse_graph_attention_amd as m

    return m


@pytest.fixture(scope="module")
def layers():
    from sparse_graph_attention_amd import layers as m

    return m


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _away_from_kink(s_src, s_dst, s_edge, src, dst, gap=0.05):
    """Shift edge terms so that |s_src[u] + s_dst[v] + s_edge[e]| >= gap - rounding."""
    z = s_src[src].astype(np.float64) + s_dst[dst] + s_edge
    near = np.abs(z) < gap
    s_edge = s_edge.copy()
    s_edge[near] += np.where(z[near] >= 0, gap, -gap).astype(np.float32)
    return s_edge


@pytest.mark.parametrize("heads,c", [(8, 8), (4, 16), (2, 3), (16, 16), (16, 32)])
def test_edge_attention(g, heads, c):
    n = 3000
    src, dst = synth.mixed_degree_graph(n, 51, hubs=(5000, 1500, 300))
    e = src.size
    rng = np.random.default_rng(heads * 100 + c)
    s_src = rng.standard_normal((n, heads)).astype(np.float32)
    s_dst = rng.standard_normal((n, heads)).astype(np.float32)
    s_edge = _away_from_kink(s_src, s_dst, rng.standard_normal((e, heads)).astype(np.float32), src, dst)
    hf = rng.standard_normal((n, heads, c)).astype(np.float32)
    d_out = rng.standard_normal((n, heads, c)).astype(np.float32)
    print(f"edge attention H={heads} C={c} n={n} e={e}", flush=True)
    topo = g.Topology(n, i32(src), i32(dst), backward=True)
    desc = g.make_desc(n, e, heads, c, g.GGA_SCORE_ADDITIVE, g.GGA_F32, 1.0, 0.2)
    out, lse = g.gga_local_attn_fwd_edge(desc, _t(s_dst), _t(s_src), _t(hf), _t(s_edge), topo)
    d_sd, d_ss, d_hf, d_se = g.gga_local_attn_bwd_edge(desc, _t(s_dst), _t(s_src), _t(hf), _t(s_edge), out, lse,
                                                       _t(d_out), topo)
    torch.cuda.synchronize()
    og = oracle.Graph(n, src, dst)
    ro, rl = oracle.local_fwd_add(s_src, s_dst, hf, og, s_edge=s_edge)
    rb = oracle.local_bwd_add(s_src, s_dst, hf, d_out, og, s_edge=s_edge)
    assert_close(out.cpu().numpy(), ro, "f32", "out")
    assert_close(lse.cpu().numpy(), rl, "f32", "lse")
    assert_close(d_sd.cpu().numpy(), rb["d_s_dst"], "f32", "d_s_dst")
    assert_close(d_ss.cpu().numpy(), rb["d_s_src"], "f32", "d_s_src")
    assert_close(d_hf.cpu().numpy(), rb["d_hf"], "f32", "d_hf")
    assert_close(d_se.cpu().numpy(), rb["d_s_edge"], "f32", "d_s_edge")


def test_edge_attention_zero_term_is_plain(g):
    """A zero edge term gives the plain additive kernels' results bit for bit."""
    n, heads, c = 2000, 8, 8
    src, dst = synth.mixed_degree_graph(n, 52, hubs=(3000, 200))
    rng = np.random.default_rng(5)
    s_src, s_dst = (_t(rng.standard_normal((n, heads))) for _ in range(2))
    hf = _t(rng.standard_normal((n, heads, c)))
    d_out = _t(rng.standard_normal((n, heads, c)))
    topo = g.Topology(n, i32(src), i32(dst), backward=True)
    desc = g.make_desc(n, src.size, heads, c, g.GGA_SCORE_ADDITIVE, g.GGA_F32, 1.0, 0.2)
    zero = torch.zeros(src.size, heads, device="cuda")
    o1, l1 = g.gga_local_attn_fwd(desc, s_dst, s_src, hf, topo.row_ptr, topo.col, topo.plan)
    o2, l2 = g.gga_local_attn_fwd_edge(desc, s_dst, s_src, hf, zero, topo)
    b1 = g.gga_local_attn_bwd(desc, s_dst, s_src, hf, o1, l1, d_out, topo)
    b2 = g.gga_local_attn_bwd_edge(desc, s_dst, s_src, hf, zero, o2, l2, d_out, topo)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for x, y in zip(b1, b2[:3]):
        assert torch.equal(x, y)


@pytest.mark.parametrize("n,heads,c", [(1000, 8, 8), (77, 3, 5), (0, 2, 4)])
def test_head_mean(g, n, heads, c):
    rng = np.random.default_rng(n + heads)
    x = rng.standard_normal((n, heads, c)).astype(np.float32)
    d = rng.standard_normal((n, c)).astype(np.float32)
    out = g.gga_head_mean(_t(x))
    d_in = g.gga_head_mean_bwd(_t(d), heads)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), x.astype(np.float64).mean(1), "f32", "mean")
    assert_close(d_in.cpu().numpy(), np.repeat(d[:, None, :] / heads, heads, axis=1), "f32", "d_in")


def _edge_features_away_from_kink(x, w, a_s, a_t, edge, src, dst, seed, thr=1e-4):
    """Re-draw the feature rows of edges whose logit (in fp64 from the fp32 inputs) lies
    within thr of the LeakyReLU kink."""
    hf, s_src, s_dst = oracle.gat_coefficients(x, w, a_s, a_t)
    heads, c = a_s.shape
    gk = np.stack([edge["w_e"][:, k * c:(k + 1) * c].astype(np.float64) @ edge["a_e"][k] for k in range(heads)], 1)
    base = s_src[src] + s_dst[dst]
    f = edge["f"].copy()
    rng = np.random.default_rng(seed)
    for _ in range(20):
        bad = np.nonzero((np.abs(base + f.astype(np.float64) @ gk) < thr).any(1))[0]
        if bad.size == 0:
            return dict(edge, f=f)
        f[bad] = rng.standard_normal((bad.size, f.shape[1])).astype(np.float32)
    raise AssertionError("could not move the logits off the kink")


def _layer_case(g, layers, n, src, dst, x, w, a_s, a_t, edge, d_out, concat):
    topo = g.Topology(n, i32(src), i32(dst), backward=True)
    ed = {k: _t(v) for k, v in edge.items()}
    f = layers.gat_forward(_t(x), _t(w), _t(a_s), _t(a_t), topo, concat=concat, edge=ed)
    b = layers.gat_backward(_t(x), _t(w), _t(a_s), _t(a_t), _t(d_out), f, topo, concat=concat, edge=ed)
    torch.cuda.synchronize()
    og = oracle.Graph(n, src, dst)
    rf = oracle.gat_forward(x, w, a_s, a_t, og, concat=concat, edge=edge)
    rb = oracle.gat_backward(x, w, a_s, a_t, d_out, og, concat=concat, edge=edge)
    assert_close(f["out"].cpu().numpy(), rf["out"], "f32", "out")
    assert_close(b["d_x"].cpu().numpy(), rb["d_x"], "f32", "d_x")
    assert_close(b["d_f"].cpu().numpy(), rb["d_f"], "f32", "d_f")
    assert_close(b["d_s_edge"].cpu().numpy(), rb["d_s_edge"], "f32", "d_s_edge")
    # sums over all nodes or edges: fp32 accumulation error grows like sqrt(count)
    big = 1e-5 * np.sqrt(max(n, src.size))
    for key in ("d_w", "d_a_s", "d_a_t", "d_w_e", "d_a_e"):
        assert_close(b[key].cpu().numpy(), rb[key], "f32", key, atol=big)


@pytest.mark.parametrize("concat", [True, False])
def test_edge_gat_layer_small(g, layers, concat):
    n, fin, heads, c, fe = 3000, 16, 4, 8, 5
    src, dst = synth.mixed_degree_graph(n, 53, hubs=(4000, 700))
    rng = np.random.default_rng(9)
    x = rng.standard_normal((n, fin)).astype(np.float32)
    w = (rng.standard_normal((fin, heads * c)) * 0.3).astype(np.float32)
    a_s, a_t, a_e = ((rng.standard_normal((heads, c)) * 0.3).astype(np.float32) for _ in range(3))
    edge = dict(f=rng.standard_normal((src.size, fe)).astype(np.float32),
                w_e=(rng.standard_normal((fe, heads * c)) * 0.3).astype(np.float32), a_e=a_e)
    edge = _edge_features_away_from_kink(x, w, a_s, a_t, edge, src, dst, 10)
    d_out = rng.standard_normal((n, heads * c if concat else c)).astype(np.float32)
    _layer_case(g, layers, n, src, dst, x, w, a_s, a_t, edge, d_out, concat)


def test_edge_gat_workload(g, layers):
    """The 170k-node power-law graph with 16 learned features per edge and heads averaged
    (forward + every first-order gradient, all rows and edges)."""
    w = synth.WORKLOADS[7]
    n = w.n
    src, dst = synth.workload_graph(7)
    print(f"workload {w.name}: n={n} e={src.size}", flush=True)
    x, wt, a_s, a_t, _ = synth.gat_inputs(n)
    edge = synth.gat_edge_inputs(src.size)
    edge = _edge_features_away_from_kink(x, wt, a_s, a_t, edge, src, dst, 11)
    d_out = synth.node_tensor(7, 0, (n, w.head_dim), stream=synth.GRADS)
    _layer_case(g, layers, n, src, dst, x, wt, a_s, a_t, edge, d_out, concat=False)
