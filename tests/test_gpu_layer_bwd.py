"""GPU parity of the backward of the gated local-global layer ("Gated Local-Global Graph
Attention", Key formulas and Implementation notes item 2) against the oracle: each new
entry point alone (LayerNorm, gate and combination, global branch, accumulating product)
over the shapes their dispatch distinguishes, then the whole layer on a small graph and on
the 262k-node layer workload, every gradient on every row.

Gradient tensors are compared with rtol 1e-4 and atol 1e-5 x RMS of the oracle's tensor:
their magnitudes range over orders (the global branch's are O(1/n), the parameter
gradients O(sqrt n)), so a fixed absolute floor would be either vacuous or unreachable."""

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


def _close(got, want, what):
    got = got.cpu().numpy() if isinstance(got, torch.Tensor) else got
    want = np.asarray(want, np.float64)
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    return assert_close(got, want, "f32", what, atol=1e-5 * rms + 1e-30)


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


@pytest.mark.parametrize("n,d", [(1000, 256), (777, 100), (300, 1024), (130, 2000), (1, 8), (0, 64)])
def test_add_layernorm_bwd(g, n, d):
    x, y, d_out = _rand((n, d), 1), _rand((n, d), 2), _rand((n, d), 3)
    gamma = 1.0 + _rand(d, 4, 0.1)
    print(f"layernorm bwd n={n} d={d}", flush=True)
    d_pre, d_gamma, d_beta = g.gga_add_layernorm_bwd(_t(x), _t(y), _t(gamma), _t(d_out), 1e-5)
    torch.cuda.synchronize()
    da, dg, db = oracle.layer_norm_bwd(x.astype(np.float64) + y, gamma, d_out, 1e-5)
    _close(d_pre, da, "d_pre")
    _close(d_gamma, dg if n else np.zeros(d), "d_gamma")
    _close(d_beta, db if n else np.zeros(d), "d_beta")


@pytest.mark.parametrize("n,d,width", [(1000, 256, 256), (513, 100, 36), (64, 64, 64), (0, 32, 32),
                                       (257, 30, 22)])  # widths off the 4-float vectors: the scalar loops
def test_gated_combine_bwd(g, n, d, width):
    x = _rand((n, d), 5)
    w_g = _rand(d, 6, 0.3)
    b_g = 0.1
    l, gl, d_y, d_in = _rand((n, width), 7), _rand((n, width), 8), _rand((n, width), 9), _rand((n, d), 10)
    print(f"combine bwd n={n} d={d} width={width}", flush=True)
    d_l, d_g, d_x, d_wg, d_bg, d_lg = g.gga_gated_combine_bwd(_t(x), _t(w_g), b_g, _t(l), _t(gl), _t(d_y), _t(d_in),
                                                              want_logit=True)
    # without an input gradient: only the logit gradients leave (the caller adds d_logit w_g^T)
    d_l2, d_g2, none, d_wg2, d_bg2, d_lg2 = g.gga_gated_combine_bwd(_t(x), _t(w_g), b_g, _t(l), _t(gl), _t(d_y),
                                                                     None)
    torch.cuda.synchronize()
    assert none is None
    gv = oracle.gate(x, w_g, b_g)
    dt = (d_y.astype(np.float64) * (l.astype(np.float64) - gl)).sum(-1) * gv * (1.0 - gv)
    _close(d_l, gv[:, None] * d_y, "d_l")
    _close(d_g, (1.0 - gv)[:, None] * d_y, "d_g")
    _close(d_x, d_in + np.outer(dt, w_g), "d_x")
    _close(d_lg, dt, "d_logit")
    _close(d_wg, x.astype(np.float64).T @ dt, "d_w_g")
    _close(d_bg, np.array([dt.sum()]), "d_b_g")
    # the two modes run the same arithmetic: identical bits
    for a, b in ((d_l, d_l2), (d_g, d_g2), (d_wg, d_wg2), (d_bg, d_bg2), (d_lg, d_lg2)):
        assert torch.equal(a, b)


def test_gated_combine_bwd_in_place(g):
    """d_x_out may be d_x_in."""
    n, d = 300, 64
    x, l, gl, d_y = _rand((n, d), 11), _rand((n, d), 12), _rand((n, d), 13), _rand((n, d), 14)
    w_g = _rand(d, 15, 0.3)
    d_in = _rand((n, d), 16)
    buf = _t(d_in)
    g.gga_gated_combine_bwd(_t(x), _t(w_g), 0.0, _t(l), _t(gl), _t(d_y), buf, d_x_out=buf)
    _, _, ref, _, _, _ = g.gga_gated_combine_bwd(_t(x), _t(w_g), 0.0, _t(l), _t(gl), _t(d_y), _t(d_in))
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)


@pytest.mark.parametrize("n,heads,r", [(1000, 4, 64), (997, 2, 48), (500, 8, 32), (77, 3, 16), (1, 1, 64),
                                       (600, 2, 24), (40, 5, 8), (300, 1, 64 - 1),
                                       (150001, 4, 64)])  # 592-row tiles, a ragged last one
def test_global_linear_bwd(g, n, heads, r):
    q, k, v = _rand((n, heads, r), 20), _rand((n, heads, r), 21), _rand((n, heads, r), 22)
    d_g = _rand((n, heads, r), 23)
    print(f"global bwd n={n} H={heads} r={r}", flush=True)
    ref = oracle.global_linear_bwd(q, k, v, d_g, 1e-6)
    names = ("d_q", "d_k", "d_v")
    qd, kd, vd, gd = _t(q), _t(k), _t(v), _t(d_g)
    s, z, gfw = g.gga_global_linear_fwd(qd, kd, vd, 1e-6)
    grads = [torch.zeros(n, heads, r, device="cuda") for _ in names]
    g.gga_global_linear_bwd(qd, kd, vd, s, z, gd, *grads, 1e-6)
    # with the forward's G the query pass reads dG . G instead of forming num again
    grads_g = [torch.zeros(n, heads, r, device="cuda") for _ in names]
    g.gga_global_linear_bwd(qd, kd, vd, s, z, gd, *grads_g, 1e-6, g_fw=gfw)
    # the kernels add into what is there: from a nonzero start the result is that start plus
    # the same contribution (the addition may be fused with the last product, so the two
    # differ by at most a rounding of each)
    base = [_t(_rand((n, heads, r), 24 + i)) for i in range(3)]
    acc = [b.clone() for b in base]
    g.gga_global_linear_bwd(qd, kd, vd, s, z, gd, *acc, 1e-6)
    torch.cuda.synchronize()
    scale = global_term_scales(q, k, v, d_g, 1e-6)
    for got, nm in zip(grads_g, names):
        assert_close(got.cpu().numpy(), ref[nm], "f32", nm + " (forward G)", atol=1e-5 * scale[nm])
    for got, b, a, nm in zip(grads, base, acc, names):
        assert_close(got.cpu().numpy(), ref[nm], "f32", nm, atol=1e-5 * scale[nm])
        lim = 2.0 ** -23 * (b.abs() + 2 * got.abs())
        assert bool(((a - (b + got)).abs() <= lim).all()), nm


@pytest.mark.parametrize("m,k,n,ta,tb", [(300, 200, 150, False, True), (256, 5000, 64, True, False),
                                         (512, 256, 256, False, False), (512, 256, 384, False, True),
                                         (64, 262144 // 16, 256, True, False), (1, 7, 3, False, False),
                                         (5003, 64, 128, False, True), (2049, 128, 64, False, False),
                                         (5000, 256, 300, False, True), (4096, 300, 257, False, True),
                                         (128, 40000, 128, True, False)])
def test_linear_accumulate(g, m, k, n, ta, tb):
    a = _rand((k, m) if ta else (m, k), 40)
    b = _rand((n, k) if tb else (k, n), 41)
    c0 = _rand((m, n), 42)
    c = _t(c0)
    g.gga_linear_accumulate(_t(a), _t(b), c, trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    op_a = a.astype(np.float64).T if ta else a.astype(np.float64)
    op_b = b.astype(np.float64).T if tb else b.astype(np.float64)
    want = c0 + op_a @ op_b
    assert_close(c.cpu().numpy(), want, "f32", "c", atol=1e-5 * np.sqrt(k))


def _dev(p):
    return {kk: (torch.from_numpy(np.ascontiguousarray(vv)).cuda() if isinstance(vv, np.ndarray) else vv)
            for kk, vv in p.items()}


def _layer(g, n, src, dst, heads, p, d_out):
    from sparse_graph_attention_amd import layers

    topo = g.Topology(n, i32(src), i32(dst), backward=True)
    pd = _dev(p)
    fwd = layers.gated_layer_forward(pd, topo, heads)
    grads = layers.gated_layer_backward(pd, fwd, topo, heads, _t(d_out))
    torch.cuda.synchronize()
    ref = oracle.gated_layer_backward(p, oracle.Graph(n, src, dst), heads, d_out)
    for name in ("d_x", "d_w_q", "d_w_k", "d_w_v", "d_w_o", "d_w_g", "d_gamma", "d_beta"):
        _close(grads[name], ref[name], name)
    _close(grads["d_b_g"], np.array([ref["d_b_g"]]), "d_b_g")


def test_layer_bwd_small(g):
    n, d, heads = 3000, 256, 4
    src, dst = synth.mixed_degree_graph(n, 33, hubs=(2000, 100))
    p = synth.gated_layer_inputs(n, d=d)
    _layer(g, n, src, dst, heads, p, _rand((n, d), 50))


def test_layer_bwd_narrow_heads(g):
    """Head width 24: the global branch's scalar path."""
    n, d, heads = 1500, 96, 4
    src, dst = synth.mixed_degree_graph(n, 34, hubs=(700, 65))
    p = synth.gated_layer_inputs(n, d=d)
    _layer(g, n, src, dst, heads, p, _rand((n, d), 51))


def test_layer_bwd_odd_width(g):
    """d = 80 (4 heads of 20): the projections' per-product paths, dX through three
    accumulating products and the separate outer-product pass, the scalar global branch."""
    n, d, heads = 1200, 80, 4
    src, dst = synth.mixed_degree_graph(n, 35, hubs=(900, 70))
    p = synth.gated_layer_inputs(n, d=d)
    _layer(g, n, src, dst, heads, p, _rand((n, d), 53))


def test_layer_bwd_workload(g):
    w = synth.WORKLOADS[4]
    n = w.n
    src, dst = synth.workload_graph(4)
    print(f"workload {w.name}: n={n} e={src.size}", flush=True)
    p = synth.gated_layer_inputs(n, d=w.d_model)
    _layer(g, n, src, dst, w.heads, p, _rand((n, w.d_model), 52))
