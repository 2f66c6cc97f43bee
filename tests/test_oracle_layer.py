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
