"""GPU parity of relation-typed messages (GiGL pull request "Support relation message modes
on the packed GraphTransformerEncoder path", section "Approach": per-relation transforms,
mean or softmax weighting, packed rows with host-side (relation, start, end) segments)
against the oracle: the packed-row mapping (bit-exact), the local kernels reading sources
from (node, relation) rows in both weightings over every degree bucket and lane layout in
fp32 and bf16, and the relation layer forward + first-order gradients on ragged batches,
an edgeless batch and the 131k-token workloads in both modes."""

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


@pytest.fixture(scope="module")
def layers():
    from sparse_graph_attention_amd import layers as m

    return m


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _random_segments(e, n_seg, n_rel, rng):
    cuts = np.sort(rng.integers(0, e + 1, n_seg - 1))
    bounds = np.concatenate([[0], cuts, [e]])
    return [(int(rng.integers(0, n_rel)), int(bounds[i]), int(bounds[i + 1])) for i in range(n_seg)]


def _by_row(t):
    """[R, N, ...] per-relation tensor -> the [N*R, ...] (node, relation) row layout."""
    return np.ascontiguousarray(np.swapaxes(t, 0, 1).reshape((-1,) + t.shape[2:]))


@pytest.mark.parametrize("n_seg", [1, 5, 100])
def test_relation_sources_bit_exact(g, n_seg):
    n, n_rel, e = 5000, 5, 60000
    rng = np.random.default_rng(n_seg)
    src = rng.integers(0, n, e).astype(np.int32)
    dst = rng.integers(0, n, e).astype(np.int32)
    src[3], src[100], dst[50] = n, -7, n + 2
    segs = _random_segments(e, n_seg, n_rel, rng)
    rel = oracle.relation_of_segments(e, segs, n_rel)
    want, bad_src = oracle.relation_rows(src, rel, n, n_rel)
    bad = bad_src + int(((dst < 0) | (dst >= n)).sum())
    got, d_bad = g.gga_relation_sources(n, n_rel, i32(src), i32(dst), segs)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), want)
    assert int(d_bad.item()) == bad == 3


def test_relation_sources_empty(g):
    e0 = torch.zeros(0, dtype=torch.int32, device="cuda")
    for segs in ([], [(0, 0, 0), (1, 0, 0)]):
        got, d_bad = g.gga_relation_sources(10, 2, e0, e0, segs)
        torch.cuda.synchronize()
        assert got.numel() == 0 and int(d_bad.item()) == 0
    with pytest.raises(g.GGAError):
        g.gga_relation_sources(10, 2, e0, e0, [(0, 0, 1)])


@pytest.mark.parametrize("mode", ["mean", "dot"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("heads,c", [(8, 8), (4, 16), (2, 3), (8, 64)])
def test_relation_attention_kernels(g, mode, dtype, heads, c):
    n, n_rel = 3000, 3
    src, dst = synth.mixed_degree_graph(n, 61, hubs=(5000, 1500, 300))
    e = src.size
    rng = np.random.default_rng(heads * 100 + c)
    rel = rng.integers(0, n_rel, e).astype(np.int32)
    rows, bad = oracle.relation_rows(src, rel, n, n_rel)
    assert bad == 0
    qh, qd = node_pair(rng.standard_normal((n, heads, c)).astype(np.float32), dtype)
    kh, kd = node_pair(_by_row(rng.standard_normal((n_rel, n, heads, c)).astype(np.float32)), dtype)
    vh, vd = node_pair(_by_row(rng.standard_normal((n_rel, n, heads, c)).astype(np.float32)), dtype)
    d_out = rng.standard_normal((n, heads, c)).astype(np.float32)
    key = np.swapaxes(kh.reshape(n, n_rel, heads, c), 0, 1)
    val = np.swapaxes(vh.reshape(n, n_rel, heads, c), 0, 1)
    print(f"relation kernels {mode} {dtype} H={heads} C={c} n={n} e={e}", flush=True)
    mean = mode == "mean"
    topo = g.Topology(n, i32(rows), i32(dst), backward=True, n_src=n * n_rel)
    desc = g.make_desc(n, e, heads, c, g.GGA_SCORE_MEAN if mean else g.GGA_SCORE_DOT,
                       g.GGA_BF16 if dtype == "bf16" else g.GGA_F32, c ** -0.5, n_src=n * n_rel)
    q_arg, k_arg = (None, None) if mean else (qd, kd)
    out, lse = g.gga_local_attn_fwd(desc, q_arg, k_arg, vd, topo.row_ptr, topo.col, topo.plan)
    if mean:
        _, _, d_v = g.gga_local_attn_bwd(desc, None, None, None, None, None, _t(d_out), topo)
    else:
        d_q, d_k, d_v = g.gga_local_attn_bwd(desc, qd, kd, vd, out, lse, _t(d_out), topo)
    torch.cuda.synchronize()
    omode = oracle.REL_MEAN if mean else oracle.REL_SOFTMAX
    ro, rl = oracle.relation_attention(None if mean else qh, None if mean else key, val, src, dst, rel, omode)
    rb = oracle.relation_attention_bwd(None if mean else qh, None if mean else key, val, d_out, src, dst, rel, omode)
    assert_close(out.cpu().numpy(), ro, dtype, "out")
    assert_close(lse.cpu().numpy(), rl, dtype, "lse")
    assert_close(d_v.cpu().numpy(), _by_row(rb["d_val"]), dtype, "d_v")
    if not mean:
        assert_close(d_q.cpu().numpy(), rb["d_q"], dtype, "d_q")
        assert_close(d_k.cpu().numpy(), _by_row(rb["d_key"]), dtype, "d_k")


def test_mean_equals_dot_with_zero_scale(g):
    """Mean weighting is the softmax of equal scores: the dot kernels at scale 0 give the
    same forward (up to rounding of the shared sums) and the same d_v."""
    n, n_rel, heads, c = 2000, 2, 4, 16
    src, dst = synth.mixed_degree_graph(n, 62, hubs=(4000, 300))
    rng = np.random.default_rng(1)
    rows, _ = oracle.relation_rows(src, rng.integers(0, n_rel, src.size), n, n_rel)
    q = _t(rng.standard_normal((n, heads, c)))
    k, v = (_t(rng.standard_normal((n * n_rel, heads, c))) for _ in range(2))
    d_out = _t(rng.standard_normal((n, heads, c)))
    topo = g.Topology(n, i32(rows), i32(dst), backward=True, n_src=n * n_rel)
    dm = g.make_desc(n, src.size, heads, c, g.GGA_SCORE_MEAN, g.GGA_F32, 1.0, n_src=n * n_rel)
    dd = g.make_desc(n, src.size, heads, c, g.GGA_SCORE_DOT, g.GGA_F32, 0.0, n_src=n * n_rel)
    o1, l1 = g.gga_local_attn_fwd(dm, None, None, v, topo.row_ptr, topo.col, topo.plan)
    o2, l2 = g.gga_local_attn_fwd(dd, q, k, v, topo.row_ptr, topo.col, topo.plan)
    _, _, dv1 = g.gga_local_attn_bwd(dm, None, None, None, None, None, d_out, topo)
    _, dk2, dv2 = g.gga_local_attn_bwd(dd, q, k, v, o2, l2, d_out, topo)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert_close(dv1.cpu().numpy(), dv2.cpu().numpy(), "f32", "d_v")
    assert not dk2.any()


def _close(got, want, what):
    got = got.cpu().numpy() if isinstance(got, torch.Tensor) else got
    want = np.asarray(want, np.float64)
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    return assert_close(got, want, "f32", what, atol=1e-5 * rms + 1e-30)


def _cat(w):
    """[R, d, W] per-relation transforms -> [d, R*W] side by side."""
    return np.concatenate(list(w), axis=1)


def _layer_case(g, layers, n, src, dst, rel, segs, p, heads, n_rel, mean):
    topo, bad = layers.relation_topology(n, n_rel, i32(src), i32(dst), segs, backward=True)
    w_q, w_k, w_v = _t(p["w_q"]), _t(_cat(p["w_k"])), _t(_cat(p["w_v"]))
    x = _t(p["x"])
    f = layers.relation_forward(x, w_q, w_k, w_v, topo, heads, n_rel, mean)
    b = layers.relation_backward(x, w_q, w_k, w_v, _t(p["d_out"]), f, topo, heads, n_rel, mean)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    mode = oracle.REL_MEAN if mean else oracle.REL_SOFTMAX
    rf = oracle.relation_forward(p["x"], p["w_q"], p["w_k"], p["w_v"], src, dst, rel, heads, mode)
    rb = oracle.relation_backward(p["x"], p["w_q"], p["w_k"], p["w_v"], src, dst, rel, heads, mode, p["d_out"])
    assert_close(f["out"].cpu().numpy(), rf["out"], "f32", "out")
    _close(b["d_x"], rb["d_x"], "d_x")
    _close(b["d_w_v"], _cat(rb["d_w_v"]), "d_w_v")
    if mean:
        assert b["d_w_q"] is None and b["d_w_k"] is None
    else:
        _close(b["d_w_q"], rb["d_w_q"], "d_w_q")
        _close(b["d_w_k"], _cat(rb["d_w_k"]), "d_w_k")


@pytest.mark.parametrize("mean", [True, False])
def test_relation_layer_ragged(g, layers, mean):
    sizes = (1, 0, 17, 300, 900, 2, 256, 0, 500, 63)
    n_rel, heads, c, d = 4, 4, 8, 48
    n, src, dst, rel, segs = synth.relation_edges(sizes, 6, n_rel, np.random.default_rng(3))
    p = synth.relation_inputs(n, d, heads, c, n_rel, ident=31)
    print(f"relation layer ragged mean={mean}: n={n} e={src.size}", flush=True)
    _layer_case(g, layers, n, src, dst, rel, segs, p, heads, n_rel, mean)


@pytest.mark.parametrize("mean", [True, False])
def test_relation_layer_no_edges(g, layers, mean):
    """An edgeless batch: no messages, zero output and zero gradients."""
    n, n_rel, heads, c, d = 100, 2, 2, 8, 16
    e0 = np.zeros(0, np.int32)
    p = synth.relation_inputs(n, d, heads, c, n_rel, ident=32)
    _layer_case(g, layers, n, e0, e0, e0, [(0, 0, 0), (1, 0, 0)], p, heads, n_rel, mean)


@pytest.mark.parametrize("ident", [8, 9])
def test_relation_workload(g, layers, ident):
    """The 512 x 256-token packed batch, d=512, 8 heads, 3 relations (every row and every
    gradient entry)."""
    w = synth.WORKLOADS[ident]
    n, src, dst, rel, segs = synth.workload_relation_edges(ident)
    print(f"workload {w.name}: n={n} e={src.size}", flush=True)
    p = synth.relation_inputs(n, w.d_model, w.heads, w.head_dim, w.relations, ident=8)
    _layer_case(g, layers, n, src, dst, rel, segs, p, w.heads, w.relations, w.score == "mean")
