"""Pins of the oracle's GAT-style additive attention, forward and backward.

- The two exact witnesses printed on the Tinymesh "Sparse attention experiment" page
  (sections "Exact single-head witness" and "Exact two-head witness"): every printed
  value is reproduced by one SGD step driven by the oracle's forward and backward.
  Float32 values printed to 6 decimals, so the oracle (fp64) must agree to 5e-7.
- Autograd (library) through a dense formulation with torch.softmax on tiny graphs.
- Shift invariance: adding a constant to s_dst[v] (every score of row v when all its
  logits are positive) leaves out unchanged and shifts lse; head permutation only
  permutes output columns (Tinymesh "Exact two-head witness").
"""

import numpy as np
import pytest
import torch

import oracle
import synth


def _witness_run(fx):
    x = np.array(fx["x"]).reshape(-1, 1)
    n = x.shape[0]
    heads = len(fx["a_s"])
    g = oracle.Graph(n, np.array(fx["src"], np.int32), np.array(fx["dst"], np.int32))
    w = np.array(fx["w"]).reshape(1, heads)
    a_s = np.array(fx["a_s"]).reshape(heads, 1)
    a_t = np.array(fx["a_t"]).reshape(heads, 1)
    node = int(fx["target_node"][0])
    target = np.array(fx["target"])

    def loss_and_grad(w, a_s, a_t):
        out = oracle.gat_forward(x, w, a_s, a_t, g)["out"]
        err = out[node] - target
        loss = float((err ** 2).mean())
        d_out = np.zeros_like(out)
        d_out[node] = 2.0 * err / heads
        return loss, oracle.gat_backward(x, w, a_s, a_t, d_out, g)

    lr = fx["lr"][0]
    l0, gr = loss_and_grad(w, a_s, a_t)
    w1 = w - lr * gr["d_w"]
    a_s1 = a_s - lr * gr["d_a_s"]
    a_t1 = a_t - lr * gr["d_a_t"]
    l1, _ = loss_and_grad(w1, a_s1, a_t1)
    return l0, gr["d_a_s"].ravel(), l1, w1.ravel(), a_s1.ravel()


@pytest.mark.parametrize("name", ["witness_single_head.txt", "witness_two_head.txt"])
def test_exact_witness(golden, name):
    fx = golden(name)
    l0, ga, l1, w1, a1 = _witness_run(fx)
    tol = 5e-7 + 1e-6  # printed to 6 decimals from float32 runs
    assert abs(l0 - fx["initial_loss"][0]) < tol
    np.testing.assert_allclose(ga, fx["grad_a_s"], atol=tol, rtol=0)
    assert abs(l1 - fx["final_loss"][0]) < tol
    np.testing.assert_allclose(w1, fx["final_w"], atol=tol, rtol=0)
    np.testing.assert_allclose(a1, fx["final_a_s"], atol=tol, rtol=0)


def test_witness_rejects_other_slopes(golden):
    """The witness is sensitive to the LeakyReLU slope: 0.2 reproduces it, 0.01 does not."""
    fx = golden("witness_single_head.txt")
    x = np.array(fx["x"]).reshape(-1, 1)
    g = oracle.Graph(3, np.array([0, 1], np.int32), np.array([2, 2], np.int32))
    one = np.ones((1, 1))
    out = oracle.gat_forward(x, one, one, np.zeros((1, 1)), g, slope=0.01)["out"]
    assert abs(float((out[2, 0] - 1.0) ** 2) - fx["initial_loss"][0]) > 1e-3


def _dense_gat(x, w, a_s, a_t, src, dst, n, slope):
    """Dense formulation with library softmax; multiplicity enters as log(count)."""
    heads, c = a_s.shape
    hf = (x @ w).reshape(n, heads, c)
    s_src = (hf * a_s[None]).sum(-1)  # [n, heads]
    s_dst = (hf * a_t[None]).sum(-1)
    cnt = torch.zeros(n, n, dtype=torch.float64)
    cnt.index_put_((torch.tensor(dst).long(), torch.tensor(src).long()), torch.ones(len(src), dtype=torch.float64),
                   accumulate=True)
    logits = s_dst.T[:, :, None] + s_src.T[:, None, :]  # [heads, v, u]
    sc = torch.nn.functional.leaky_relu(logits, slope) + torch.log(cnt)[None]
    alpha = torch.softmax(sc, dim=-1)
    out = torch.einsum("hvu,uhc->vhc", alpha, hf)
    return out.reshape(n, heads * c)


@pytest.mark.parametrize("n,m,seed,heads,c", [(3, 4, 0, 1, 2), (10, 40, 1, 2, 3), (30, 200, 2, 4, 2)])
def test_gat_fwd_bwd_match_dense_autograd(n, m, seed, heads, c):
    src, dst = synth.random_multigraph(n, m, seed, self_loops=True)
    g = oracle.Graph(n, src, dst)
    rng = np.random.default_rng(seed)
    fin = 5
    x = rng.standard_normal((n, fin))
    w = rng.standard_normal((fin, heads * c)) * 0.5
    a_s = rng.standard_normal((heads, c))
    a_t = rng.standard_normal((heads, c))
    d_out = rng.standard_normal((n, heads * c))
    f = oracle.gat_forward(x, w, a_s, a_t, g)
    b = oracle.gat_backward(x, w, a_s, a_t, d_out, g)
    tx, tw, ts, tt = (torch.tensor(a).requires_grad_(True) for a in (x, w, a_s, a_t))
    out = _dense_gat(tx, tw, ts, tt, src, dst, n, oracle.SLOPE)
    np.testing.assert_allclose(f["out"], out.detach().numpy(), rtol=1e-12, atol=1e-12)
    (out * torch.tensor(d_out)).sum().backward()
    np.testing.assert_allclose(b["d_x"], tx.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["d_w"], tw.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["d_a_s"], ts.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["d_a_t"], tt.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_additive_shift_and_head_permutation():
    n, heads, c = 25, 3, 2
    src, dst = synth.random_multigraph(n, 120, 5, self_loops=True, isolated=2)
    g = oracle.Graph(n, src, dst)
    rng = np.random.default_rng(3)
    s_src = rng.standard_normal((n, heads)) + 50.0  # every logit positive: LeakyReLU is the identity
    s_dst = rng.standard_normal((n, heads)) + 50.0
    hf = rng.standard_normal((n, heads, c))
    out, lse = oracle.local_fwd_add(s_src, s_dst, hf, g)
    out2, lse2 = oracle.local_fwd_add(s_src, s_dst + 7.0, hf, g)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-13)
    live = np.diff(g.row_ptr) > 0
    np.testing.assert_allclose(lse2[live], lse[live] + 7.0, rtol=1e-14)
    hp = np.array([1, 2, 0])
    out3, _ = oracle.local_fwd_add(s_src[:, hp], s_dst[:, hp], hf[:, hp], g)
    np.testing.assert_array_equal(out3, out[:, hp])
    assert np.all(out[~live] == 0.0) and np.all(np.isneginf(lse[~live]))
