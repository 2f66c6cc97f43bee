"""GPU parity of the dense steps: the fp32 MFMA product, the global linear branch, the
node gate / combination and the residual LayerNorm, against the oracle (fp64)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import sparse_graph_attention_amd as m

    return m


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@pytest.mark.parametrize("m,k,n,ta,tb,bias", [
    (1, 1, 1, 0, 0, False), (7, 5, 3, 0, 0, True), (128, 128, 128, 0, 0, False), (300, 257, 130, 0, 0, True),
    (300, 257, 130, 1, 0, False), (300, 257, 130, 0, 1, True), (300, 257, 130, 1, 1, False),
    (128, 170000, 64, 1, 0, False),   # X^T dH of the GAT workload: split over k
    (170000, 64, 128, 0, 1, False),   # dH W^T
    (4096, 256, 256, 0, 0, False), (33, 0, 17, 0, 0, True),
    # whole 128 x 128 tiles and 32-deep stages (the unguarded loop), every transpose, bias
    # added through the 16-byte epilogue; ragged tiles with 16-byte rows; split k with bias
    (512, 512, 256, 0, 0, True), (512, 512, 256, 1, 1, True), (256, 384, 384, 1, 0, True),
    (384, 96, 256, 0, 1, True), (129, 33, 132, 0, 0, True), (256, 70000, 192, 1, 0, True),
    # whole k stages with ragged m and n: the fast kernel takes the inner tiles, the guarded one the edges
    (1000, 256, 300, 0, 0, True), (1000, 256, 300, 0, 1, False), (1000, 256, 300, 1, 0, True), (1000, 256, 300, 1, 1, False),
    # tall a times a small b stored [n, k]: b transposed into the workspace first
    (5000, 256, 300, 0, 1, True), (4096, 300, 257, 0, 1, False), (8192, 512, 512, 0, 1, True),
    # skinny shapes: narrow contractions (k, n <= 64) and few outputs over a long k
    (100000, 16, 8, 0, 0, True), (50000, 8, 16, 0, 1, False), (3000, 64, 64, 1, 0, True), (5, 1, 1, 0, 0, False),
    (16, 300000, 8, 1, 0, False), (32, 20000, 32, 1, 1, True), (3, 5000, 2, 0, 0, False),
    (32, 20000, 32, 1, 0, True), (7, 9000, 30, 1, 0, False), (100000, 16, 8, 1, 0, False), (999, 33, 64, 0, 1, True),
    # a thread per output row (k, n <= 32) with odd widths; one MFMA tile over a long k
    (70001, 7, 5, 0, 0, True), (4099, 32, 32, 0, 1, True), (5, 50001, 3, 1, 0, True), (16, 9000, 16, 1, 0, False),
    # op(b) held in LDS, 16-row tiles streamed (k, n <= 128): the GAT X W, ragged rows, both b layouts
    (170000, 128, 64, 0, 0, False), (4099, 96, 80, 0, 1, True), (1030, 16, 128, 0, 0, True), (2055, 128, 16, 0, 1, False),
    (2000, 0, 80, 0, 0, True),  # empty contraction beside the streaming shapes: c is the bias
    # transposed a over a long k (split-k), ragged k, with bias
    (128, 170001, 64, 1, 0, True), (48, 20000, 64, 1, 0, False), (64, 16384, 112, 1, 0, True),
    # few outputs over a long k with a transposed a: split k at every tile count of m and n in
    # {32, 64, 128}, k at and just past 4096, ragged k ranges, a k of two million
    (32, 4096, 32, 1, 0, True), (32, 5000, 64, 1, 0, False), (32, 9001, 128, 1, 0, True), (64, 4097, 32, 1, 0, False),
    (64, 33333, 64, 1, 0, True), (64, 6000, 128, 1, 0, False), (128, 12345, 32, 1, 0, True),
    (128, 4100, 64, 1, 0, False), (128, 2100000, 64, 1, 0, False),
])
def test_linear(g, m, k, n, ta, tb, bias):
    print(f"linear m={m} k={k} n={n} ta={ta} tb={tb}", flush=True)
    rng = np.random.default_rng(m + k + n)
    a = rng.standard_normal((k, m) if ta else (m, k)).astype(np.float32)
    b = rng.standard_normal((n, k) if tb else (k, n)).astype(np.float32)
    bv = rng.standard_normal(n).astype(np.float32) if bias else None
    c = g.gga_linear(_t(a), _t(b), None if bv is None else _t(bv), trans_a=bool(ta), trans_b=bool(tb))
    torch.cuda.synchronize()
    ref = (a.T if ta else a).astype(np.float64) @ (b.T if tb else b).astype(np.float64)
    if bv is not None:
        ref = ref + bv
    # fp32 accumulation over k terms of size ~1: allow sqrt(k) growth of the absolute error
    assert_close(c.cpu().numpy(), ref, "f32", "c", atol=1e-5 * max(1.0, np.sqrt(k)))


def test_linear_split_k_accumulate(g):
    """c += a^T b over a long k: the split-k partials are added into c in a fixed order."""
    rng = np.random.default_rng(5)
    a, b = rng.standard_normal((70000, 128)).astype(np.float32), rng.standard_normal((70000, 64)).astype(np.float32)
    c0 = rng.standard_normal((128, 64)).astype(np.float32)
    acc = _t(c0)
    g.gga_linear_accumulate(_t(a), _t(b), acc, trans_a=True)
    torch.cuda.synchronize()
    ref = a.T.astype(np.float64) @ b.astype(np.float64) + c0
    assert_close(acc.cpu().numpy(), ref, "f32", "c+=", atol=1e-5 * np.sqrt(70000))


def test_linear_deterministic(g):
    rng = np.random.default_rng(3)
    a, b = _t(rng.standard_normal((50000, 128))), _t(rng.standard_normal((50000, 64)))
    c1 = g.gga_linear(a, b, trans_a=True)
    c2 = g.gga_linear(a, b, trans_a=True)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


@pytest.mark.parametrize("n,h,r", [(1, 1, 16), (1000, 2, 16), (5000, 4, 64), (3001, 3, 32), (777, 2, 48),
                                   (2000, 8, 64), (3000, 12, 16),
                                   (500, 2, 5), (20000, 1, 8),
                                   # tiles longer than 256 rows: 592 at 4 heads, 272 at one head
                                   (150001, 4, 64), (270001, 1, 16)])
def test_global_linear(g, n, h, r):
    print(f"global n={n} h={h} r={r}", flush=True)
    rng = np.random.default_rng(n + r)
    q, k, v = (rng.standard_normal((n, h, r)).astype(np.float32) * 0.5 for _ in range(3))
    s, z, gg = g.gga_global_linear_fwd(_t(q), _t(k), _t(v), 1e-6)
    torch.cuda.synchronize()
    rs, rz, rg = oracle.global_linear(q, k, v, 1e-6)
    assert_close(s.cpu().numpy(), rs, "f32", "S", atol=1e-5 * np.sqrt(n))
    assert_close(z.cpu().numpy(), rz, "f32", "z", atol=1e-5 * np.sqrt(n))
    assert_close(gg.cpu().numpy(), rg, "f32", "G")


@pytest.mark.parametrize("n,d,heads", [(1000, 256, 4), (3000, 384, 4), (77, 100, 4), (5, 8, 2)])
def test_qkv_gate_projection(g, n, d, heads):
    """[Q | K | V | gate logit] = X [W_Q | W_K | W_V | w_g] + b_g: one launch for d a multiple
    of 128 (ragged row tiles included), the per-product path otherwise."""
    rng = np.random.default_rng(n + d)
    x = rng.standard_normal((n, d)).astype(np.float32)
    ws = [(rng.standard_normal((d, d)) * 0.05).astype(np.float32) for _ in range(3)]
    wg = (rng.standard_normal(d) * 0.1).astype(np.float32)
    q, k, v, logit = g.gga_qkv_gate_proj(_t(x), *(_t(w) for w in ws), _t(wg), 0.25, heads)
    torch.cuda.synchronize()
    x64 = x.astype(np.float64)
    for got, w in zip((q, k, v), ws):
        assert_close(got.reshape(n, d).cpu().numpy(), x64 @ w, "f32", "projection", atol=1e-5 * np.sqrt(d))
    assert_close(logit.cpu().numpy(), x64 @ wg + 0.25, "f32", "gate logit", atol=1e-5 * np.sqrt(d))


@pytest.mark.parametrize("n,d", [(3000, 256), (1000, 128), (77, 100)])
def test_qkv_projection_input_gradient(g, n, d):
    """d_x += dQ W_Q^T + dK W_K^T + dV W_V^T, one launch (k ranges q, k, v) or three."""
    rng = np.random.default_rng(7 * n + d)
    grads = [rng.standard_normal((n, d)).astype(np.float32) for _ in range(3)]
    ws = [(rng.standard_normal((d, d)) * 0.05).astype(np.float32) for _ in range(3)]
    dx0 = rng.standard_normal((n, d)).astype(np.float32)
    dx = _t(dx0)
    g.gga_qkv_proj_bwd_x(*(_t(a) for a in grads), *(_t(w) for w in ws), dx)
    torch.cuda.synchronize()
    want = dx0.astype(np.float64) + sum(a.astype(np.float64) @ w.T.astype(np.float64) for a, w in zip(grads, ws))
    assert_close(dx.cpu().numpy(), want, "f32", "d_x", atol=1e-5 * np.sqrt(3 * d))
    # with the gate logit's share: + d_logit w_g^T in the same call (the product's epilogue, or
    # a separate pass after the three products)
    d_logit = rng.standard_normal(n).astype(np.float32)
    w_g = (rng.standard_normal(d) * 0.1).astype(np.float32)
    dx = _t(dx0)
    g.gga_qkv_proj_bwd_x(*(_t(a) for a in grads), *(_t(w) for w in ws), dx, d_logit=_t(d_logit), w_g=_t(w_g))
    torch.cuda.synchronize()
    want = want + np.outer(d_logit.astype(np.float64), w_g)
    assert_close(dx.cpu().numpy(), want, "f32", "d_x with d_logit", atol=1e-5 * np.sqrt(3 * d + 1))


def test_gate_combine_and_limits(g):
    rng = np.random.default_rng(5)
    n, d, w = 1000, 256, 256
    x = rng.standard_normal((n, d)).astype(np.float32)
    wg = (rng.standard_normal(d) * 0.1).astype(np.float32)
    wz = np.zeros((d, d), np.float32)
    loc, glob = rng.standard_normal((n, w)).astype(np.float32), rng.standard_normal((n, w)).astype(np.float32)
    for b_g in (0.3, 80.0, -80.0):
        *_, logit = g.gga_qkv_gate_proj(_t(x), _t(wz), _t(wz), _t(wz), _t(wg), b_g, 4)
        gate, y = g.gga_gated_combine(logit, _t(loc), _t(glob))
        torch.cuda.synchronize()
        rg = oracle.gate(x, wg, b_g)
        assert_close(gate.cpu().numpy(), rg, "f32", "gate")
        assert_close(y.cpu().numpy(), oracle.combine(rg, loc, glob), "f32", "y")
    # odd widths take the scalar path
    x2 = rng.standard_normal((37, 5)).astype(np.float32)
    wg2 = rng.standard_normal(5).astype(np.float32)
    l2, g2 = rng.standard_normal((37, 3)).astype(np.float32), rng.standard_normal((37, 3)).astype(np.float32)
    logit2 = _t(x2.astype(np.float64) @ wg2.astype(np.float64) - 0.2)
    gate, y = g.gga_gated_combine(logit2, _t(l2), _t(g2))
    torch.cuda.synchronize()
    rg = oracle.gate(x2, wg2, -0.2)
    assert_close(y.cpu().numpy(), oracle.combine(rg, l2, g2), "f32", "y")


@pytest.mark.parametrize("n,d", [(1, 4), (1000, 256), (333, 1024), (50, 100), (10, 3000)])
def test_add_layernorm(g, n, d):
    rng = np.random.default_rng(n + d)
    x = (rng.standard_normal((n, d)) * 2 + 1).astype(np.float32)
    y = rng.standard_normal((n, d)).astype(np.float32)
    gm, bt = rng.standard_normal(d).astype(np.float32), rng.standard_normal(d).astype(np.float32)
    out = g.gga_add_layernorm(_t(x), _t(y), _t(gm), _t(bt), 1e-5)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), oracle.layer_norm(x.astype(np.float64) + y, gm, bt), "f32", "ln")


def test_linear_shape_sweep(g):
    """Every product path, chosen by shape and transposes (short rows, narrow, LDS-resident
    b, the tile kernels, split k), at the boundaries of the conditions that pick it: k and n
    around 16, 32, 64 and 128, an empty contraction, m below and above the streaming
    threshold, with bias and accumulation."""
    edges = (0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 80, 127, 128, 129)
    rng = np.random.default_rng(11)
    checked = 0
    for m in (37, 1030):
        for k in edges:
            for n in edges[1:]:
                for ta, tb in ((0, 0), (0, 1), (1, 0), (1, 1)):
                    a = rng.standard_normal((k, m) if ta else (m, k)).astype(np.float32)
                    b = rng.standard_normal((n, k) if tb else (k, n)).astype(np.float32)
                    bv = rng.standard_normal(n).astype(np.float32)
                    c0 = rng.standard_normal((m, n)).astype(np.float32)
                    ref = (a.T if ta else a).astype(np.float64) @ (b.T if tb else b).astype(np.float64)
                    c = g.gga_linear(_t(a), _t(b), _t(bv), trans_a=bool(ta), trans_b=bool(tb))
                    acc = _t(c0)
                    g.gga_linear_accumulate(_t(a), _t(b), acc, trans_a=bool(ta), trans_b=bool(tb))
                    torch.cuda.synchronize()
                    what = f"m={m} k={k} n={n} ta={ta} tb={tb}"
                    assert_close(c.cpu().numpy(), ref + bv, "f32", "c " + what, atol=1e-5 * max(1.0, np.sqrt(k)))
                    assert_close(acc.cpu().numpy(), ref + c0, "f32", "c+= " + what,
                                 atol=1e-5 * max(1.0, np.sqrt(k)))
                    checked += 1
    assert checked == 2 * 15 * 14 * 4
