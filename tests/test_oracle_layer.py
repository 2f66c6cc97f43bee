"""Pins of the oracle's global linear branch, gate, combine and LayerNorm.

- Global branch ("Gated Local-Global Graph Attention", Key formulas, G_i): the oracle
  factors through S and z; the pin is the dense O(N^2) kernelised form
  (phi(Q) phi(K)^T V) / (phi(Q) phi(K)^T 1 + eps), the other association (the page's
  MVP check compares exactly these two, to below 2.4e-7), with phi from torch's elu.
- Gate limits: b_g -> +inf gives Y = L, b_g -> -inf gives Y = G, w_g = b_g = 0 gives the
  mean (Key formulas, g_i = sigmoid(x_i w_g + b_g)).
- LayerNorm against torch.nn.functional.layer_norm (library).
- The assembled layer against a step-by-step torch float64 evaluation of the
  Implementation notes pseudocode on a small graph, with torch's masked softmax.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


def test_phi_matches_elu_plus_one():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.phi(x), F.elu(torch.tensor(x)).numpy() + 1.0, rtol=1e-15, atol=1e-15)
    assert np.all(oracle.phi(x) > 0)


@pytest.mark.parametrize("n,h,r", [(1, 1, 1), (17, 2, 5), (200, 4, 16)])
def test_global_matches_dense_kernelised_form(n, h, r):
    rng = np.random.default_rng(n)
    q, k, v = (rng.standard_normal((n, h, r)) for _ in range(3))
    s, z, g = oracle.global_linear(q, k, v, eps=1e-6)
    tq, tk, tv = (torch.tensor(a).permute(1, 0, 2) for a in (q, k, v))
    pq, pk = F.elu(tq) + 1, F.elu(tk) + 1
    a = pq @ pk.transpose(1, 2)  # [h, n, n]
    ref = (a @ tv) / (a.sum(-1, keepdim=True) + 1e-6)
    np.testing.assert_allclose(g, ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-13)
    # statistics are independent of node order
    p = rng.permutation(n)
    s2, z2, g2 = oracle.global_linear(q[p], k[p], v[p], eps=1e-6)
    np.testing.assert_allclose(s2, s, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z2, z, rtol=1e-12)
    np.testing.assert_allclose(g2, g[p], rtol=1e-12, atol=1e-14)


def test_gate_limits():
    rng = np.random.default_rng(0)
    n, d = 10, 6
    x = rng.standard_normal((n, d))
    w_g = rng.standard_normal(d) * 0.1
    loc, glob = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    np.testing.assert_allclose(oracle.combine(oracle.gate(x, w_g, 1e3), loc, glob), loc, rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.combine(oracle.gate(x, w_g, -1e3), loc, glob), glob, rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.combine(oracle.gate(x, 0 * w_g, 0.0), loc, glob), (loc + glob) / 2,
                               rtol=1e-15)
    np.testing.assert_allclose(oracle.gate(x, w_g, 0.3), torch.sigmoid(torch.tensor(x @ w_g + 0.3)).numpy(),
                               rtol=1e-15)


def test_layer_norm_matches_library():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((7, 256)) * 3 + 1
    gam, bet = rng.standard_normal(256), rng.standard_normal(256)
    ref = F.layer_norm(torch.tensor(a), (256,), torch.tensor(gam), torch.tensor(bet), eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.layer_norm(a, gam, bet), ref, rtol=1e-12, atol=1e-12)


def test_gated_layer_matches_stepwise_torch():
    n, d, heads = 48, 16, 4
    r = d // heads
    src, dst = synth.random_multigraph(n, 300, 4, self_loops=True)
    g = oracle.Graph(n, src, dst)
    p = synth.gated_layer_inputs(n, d=d)
    out = oracle.gated_layer(p, g, heads)
    t = {k: torch.tensor(np.asarray(v), dtype=torch.float64) for k, v in p.items()}
    x = t["x"]
    q = (x @ t["w_q"]).reshape(n, heads, r).permute(1, 0, 2)
    k = (x @ t["w_k"]).reshape(n, heads, r).permute(1, 0, 2)
    v = (x @ t["w_v"]).reshape(n, heads, r).permute(1, 0, 2)
    cnt = torch.zeros(n, n, dtype=torch.float64)
    cnt.index_put_((torch.tensor(dst).long(), torch.tensor(src).long()), torch.ones(len(src), dtype=torch.float64),
                   accumulate=True)
    loc = F.scaled_dot_product_attention(q, k, v, attn_mask=torch.log(cnt)).permute(1, 0, 2).reshape(n, d)
    pq, pk = F.elu(q) + 1, F.elu(k) + 1
    s = pk.transpose(1, 2) @ v
    z = pk.sum(1)
    glob = ((pq @ s) / ((pq * z[:, None, :]).sum(-1, keepdim=True) + 1e-6)).permute(1, 0, 2).reshape(n, d)
    gt = torch.sigmoid(x @ t["w_g"] + t["b_g"])[:, None]
    y = gt * loc + (1 - gt) * glob
    ref = F.layer_norm(x + y @ t["w_o"], (d,), t["gamma"], t["beta"], eps=1e-5)
    np.testing.assert_allclose(out["local"], loc.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(out["glob"], glob.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(out["out"], ref.numpy(), rtol=1e-10, atol=1e-11)
    rows = np.array([5, 0, 47], np.int32)
    sub = oracle.gated_layer(p, g, heads, rows=rows)
    np.testing.assert_allclose(sub["out"], out["out"][rows], rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------- layer backward


def _torch_layer(p, src, dst, n, heads, eps=1e-6):
    """The layer forward in torch float64 with a masked dense local branch (library softmax)."""
    d = p["x"].shape[1]
    r = d // heads
    t = {k: (v if isinstance(v, torch.Tensor) else torch.tensor(np.asarray(v), dtype=torch.float64))
         for k, v in p.items()}
    x = t["x"]
    q = (x @ t["w_q"]).reshape(n, heads, r).permute(1, 0, 2)
    k = (x @ t["w_k"]).reshape(n, heads, r).permute(1, 0, 2)
    v = (x @ t["w_v"]).reshape(n, heads, r).permute(1, 0, 2)
    cnt = torch.zeros(n, n, dtype=torch.float64)
    cnt.index_put_((torch.tensor(dst).long(), torch.tensor(src).long()), torch.ones(len(src), dtype=torch.float64),
                   accumulate=True)
    loc = F.scaled_dot_product_attention(q, k, v, attn_mask=torch.log(cnt)).permute(1, 0, 2).reshape(n, d)
    pq, pk = F.elu(q) + 1, F.elu(k) + 1
    s = pk.transpose(1, 2) @ v
    z = pk.sum(1)
    glob = ((pq @ s) / ((pq * z[:, None, :]).sum(-1, keepdim=True) + eps)).permute(1, 0, 2).reshape(n, d)
    gt = torch.sigmoid(x @ t["w_g"] + t["b_g"])[:, None]
    y = gt * loc + (1 - gt) * glob
    return F.layer_norm(x + y @ t["w_o"], (d,), t["gamma"], t["beta"], eps=1e-5)


def test_global_bwd_matches_autograd():
    rng = np.random.default_rng(3)
    n, h, r = 40, 2, 6
    q, k, v, dg = (rng.standard_normal((n, h, r)) for _ in range(4))
    res = oracle.global_linear_bwd(q, k, v, dg)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    pq, pk = F.elu(tq) + 1, F.elu(tk) + 1
    s = torch.einsum("nhi,nhj->hij", pk, tv)
    z = pk.sum(0)
    gg = torch.einsum("nhi,hij->nhj", pq, s) / (torch.einsum("nhi,hi->nh", pq, z) + 1e-6)[..., None]
    (gg * torch.tensor(dg)).sum().backward()
    for name, tt in (("d_q", tq), ("d_k", tk), ("d_v", tv)):
        np.testing.assert_allclose(res[name], tt.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def test_layer_norm_bwd_matches_autograd():
    rng = np.random.default_rng(4)
    a = rng.standard_normal((9, 32)) * 2 + 0.5
    gam, bet, do = rng.standard_normal(32), rng.standard_normal(32), rng.standard_normal((9, 32))
    da, dgam, dbet = oracle.layer_norm_bwd(a, gam, do)
    ta, tg, tb = (torch.tensor(z, requires_grad=True) for z in (a, gam, bet))
    (F.layer_norm(ta, (32,), tg, tb, eps=1e-5) * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(da, ta.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dgam, tg.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dbet, tb.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_gated_layer_bwd_matches_autograd():
    n, d, heads = 30, 16, 4
    src, dst = synth.random_multigraph(n, 150, 8, self_loops=True)
    g = oracle.Graph(n, src, dst)
    p = synth.gated_layer_inputs(n, d=d)
    rng = np.random.default_rng(5)
    p["gamma"] = (1 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    p["beta"] = (0.2 * rng.standard_normal(d)).astype(np.float32)
    d_out = rng.standard_normal((n, d))
    res = oracle.gated_layer_backward(p, g, heads, d_out)
    t = {k: torch.tensor(np.asarray(v), dtype=torch.float64, requires_grad=True) for k, v in p.items()}
    out = _torch_layer(t, src, dst, n, heads)
    np.testing.assert_allclose(res["fwd"]["out"], out.detach().numpy(), rtol=1e-10, atol=1e-11)
    (out * torch.tensor(d_out)).sum().backward()
    for key, name in (("d_x", "x"), ("d_w_q", "w_q"), ("d_w_k", "w_k"), ("d_w_v", "w_v"), ("d_w_o", "w_o"),
                      ("d_w_g", "w_g"), ("d_b_g", "b_g"), ("d_gamma", "gamma"), ("d_beta", "beta")):
        np.testing.assert_allclose(np.asarray(res[key]), t[name].grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=key)


def test_gated_layer_bwd_finite_differences():
    n, d, heads = 12, 8, 2
    src, dst = synth.random_multigraph(n, 40, 9, self_loops=True)
    g = oracle.Graph(n, src, dst)
    p = {k: (np.asarray(v, np.float64) if isinstance(v, np.ndarray) else v)
         for k, v in synth.gated_layer_inputs(n, d=d).items()}
    p["w_q"] = p["w_q"] * 10  # scores of order one, so every term of the layer matters
    p["w_k"] = p["w_k"] * 10
    d_out = np.random.default_rng(6).standard_normal((n, d))
    res = oracle.gated_layer_backward(p, g, heads, d_out)

    def loss(pp):
        return float((oracle.gated_layer(pp, g, heads)["out"] * d_out).sum())

    h = 1e-6
    for name, key in (("x", "d_x"), ("w_q", "d_w_q"), ("w_o", "d_w_o"), ("w_g", "d_w_g")):
        for idx in [(0, 0), (3, 1), (7, 5)] if p[name].ndim == 2 else [(0,), (5,)]:
            pp = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
            pp[name][idx] += h
            lp = loss(pp)
            pp[name][idx] -= 2 * h
            lm = loss(pp)
            assert abs((lp - lm) / (2 * h) - res[key][idx]) < 1e-6, (name, idx)
    pp = dict(p)
    pp["b_g"] = p["b_g"] + h
    lp = loss(pp)
    pp["b_g"] = p["b_g"] - h
    lm = loss(pp)
    assert abs((lp - lm) / (2 * h) - res["d_b_g"]) < 1e-6
