"""Pins of the oracle's batched (packed multi-graph) path: a batch of graphs, one adjacency
list each ("Gated Local-Global Graph Attention", Implementation notes note 1: batched X).

- batch_edges against the block-diagonal assembly of the per-graph adjacency count
  matrices (scipy.linalg.block_diag, library);
- the per-graph global branch against the dense kernelised form with a same-graph mask
  (the other association, restricted to pairs in one graph), and its backward against torch
  autograd through that form;
- the batched layer, forward and backward, against the step-by-step torch float64 layer
  with the same masks.
"""

import numpy as np
import pytest
import scipy.linalg
import torch
import torch.nn.functional as F

import oracle
import synth


def _dense_counts(n, src, dst):
    a = np.zeros((n, n))
    np.add.at(a, (dst, src), 1.0)
    return a


def test_batch_edges_is_block_diagonal():
    sizes = (3, 0, 5, 1, 4)
    node_ptr, edge_ptr, sl, dl = synth.batch_of_graphs(sizes, 3, np.random.default_rng(1))
    src, dst, bad = oracle.batch_edges(node_ptr, edge_ptr, sl, dl)
    assert bad == 0
    blocks = [_dense_counts(nb, sl[edge_ptr[b]:edge_ptr[b + 1]], dl[edge_ptr[b]:edge_ptr[b + 1]])
              for b, nb in enumerate(sizes)]
    want = scipy.linalg.block_diag(*[blk for blk in blocks if blk.size] or [np.zeros((0, 0))])
    np.testing.assert_array_equal(_dense_counts(sum(sizes), src, dst), want)
    # COO order is kept: entry i of the packed list is entry i of the batch
    assert src.shape == sl.shape
    gid = np.searchsorted(edge_ptr, np.arange(sl.size), side="right") - 1
    np.testing.assert_array_equal(src - node_ptr[gid], sl)


def test_batch_edges_flags_foreign_ids():
    node_ptr = np.array([0, 2, 5], np.int32)
    edge_ptr = np.array([0, 2, 4], np.int32)
    sl = np.array([0, 2, 1, -1], np.int32)  # 2 is outside graph 0; -1 is outside graph 1
    dl = np.array([1, 0, 3, 2], np.int32)  # 3 is outside graph 1
    src, dst, bad = oracle.batch_edges(node_ptr, edge_ptr, sl, dl)
    assert bad == 3
    np.testing.assert_array_equal(src, [0, -1, 3, -1])
    np.testing.assert_array_equal(dst, [1, 0, -1, 4])


def _masked_dense_global(tq, tk, tv, mask, eps=1e-6):
    """(phi(Q) phi(K)^T * M) V / ((phi(Q) phi(K)^T * M) 1 + eps), per head ([h, n, r])."""
    pq, pk = F.elu(tq) + 1, F.elu(tk) + 1
    a = (pq @ pk.transpose(1, 2)) * mask
    return (a @ tv) / (a.sum(-1, keepdim=True) + eps)


def _same_graph(node_ptr):
    n = int(node_ptr[-1])
    gid = np.searchsorted(node_ptr, np.arange(n), side="right") - 1
    return torch.tensor((gid[:, None] == gid[None, :]).astype(np.float64))


@pytest.mark.parametrize("sizes", [(7,), (5, 0, 9, 1), (1, 1, 1), (0, 12)])
def test_global_seg_matches_masked_dense(sizes):
    node_ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    n, h, r = int(node_ptr[-1]), 2, 5
    rng = np.random.default_rng(len(sizes))
    q, k, v = (rng.standard_normal((n, h, r)) for _ in range(3))
    s, z, g = oracle.global_linear_seg(q, k, v, node_ptr)
    tq, tk, tv = (torch.tensor(a).permute(1, 0, 2) for a in (q, k, v))
    ref = _masked_dense_global(tq, tk, tv, _same_graph(node_ptr)).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(g, ref, rtol=1e-11, atol=1e-13)
    assert s.shape == (len(sizes), h, r, r) and z.shape == (len(sizes), h, r)
    for b, nb in enumerate(sizes):
        if nb == 0:
            assert not s[b].any() and not z[b].any()


def test_global_seg_bwd_matches_autograd():
    sizes = (6, 0, 11, 1)
    node_ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    n, h, r = int(node_ptr[-1]), 2, 4
    rng = np.random.default_rng(8)
    q, k, v, dg = (rng.standard_normal((n, h, r)) for _ in range(4))
    res = oracle.global_linear_seg_bwd(q, k, v, dg, node_ptr)
    tq, tk, tv = (torch.tensor(a).permute(1, 0, 2).contiguous().requires_grad_() for a in (q, k, v))
    g = _masked_dense_global(tq, tk, tv, _same_graph(node_ptr))
    (g * torch.tensor(dg).permute(1, 0, 2)).sum().backward()
    for name, tt in (("d_q", tq), ("d_k", tk), ("d_v", tv)):
        np.testing.assert_allclose(res[name], tt.grad.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=name)


def _torch_batched_layer(t, src, dst, node_ptr, heads, eps=1e-6):
    """The layer in torch float64: masked dense local branch over the packed graph (library
    softmax) and the per-graph global branch as the masked dense form."""
    x = t["x"]
    n, d = x.shape
    r = d // heads
    q, k, v = ((x @ t[w]).reshape(n, heads, r).permute(1, 0, 2) for w in ("w_q", "w_k", "w_v"))
    cnt = torch.tensor(_dense_counts(n, src, dst))
    loc = F.scaled_dot_product_attention(q, k, v, attn_mask=torch.log(cnt)).permute(1, 0, 2).reshape(n, d)
    glob = _masked_dense_global(q, k, v, _same_graph(node_ptr), eps).permute(1, 0, 2).reshape(n, d)
    gt = torch.sigmoid(x @ t["w_g"] + t["b_g"])[:, None]
    y = gt * loc + (1 - gt) * glob
    return F.layer_norm(x + y @ t["w_o"], (d,), t["gamma"], t["beta"], eps=1e-5)


def test_batched_layer_forward_and_backward_match_torch():
    sizes = (9, 1, 0, 14)
    d, heads = 8, 2
    node_ptr, edge_ptr, sl, dl = synth.batch_of_graphs(sizes, 3, np.random.default_rng(2))
    src, dst, bad = oracle.batch_edges(node_ptr, edge_ptr, sl, dl)
    assert bad == 0
    n = int(node_ptr[-1])
    g = oracle.Graph(n, src, dst)
    p = {kk: (np.asarray(vv, np.float64) if isinstance(vv, np.ndarray) else vv)
         for kk, vv in synth.gated_layer_inputs(n, d=d).items()}
    p["w_q"] = p["w_q"] * 10
    p["w_k"] = p["w_k"] * 10
    p["w_v"] = p["w_v"] * 10
    d_out = np.random.default_rng(3).standard_normal((n, d))
    res = oracle.gated_layer_backward(p, g, heads, d_out, node_ptr=node_ptr)
    t = {kk: torch.tensor(np.asarray(vv), dtype=torch.float64, requires_grad=True) for kk, vv in p.items()}
    out = _torch_batched_layer(t, src, dst, node_ptr, heads)
    np.testing.assert_allclose(res["fwd"]["out"], out.detach().numpy(), rtol=1e-10, atol=1e-11)
    (out * torch.tensor(d_out)).sum().backward()
    for key, name in (("d_x", "x"), ("d_w_q", "w_q"), ("d_w_k", "w_k"), ("d_w_v", "w_v"), ("d_w_o", "w_o"),
                      ("d_w_g", "w_g"), ("d_b_g", "b_g"), ("d_gamma", "gamma"), ("d_beta", "beta")):
        np.testing.assert_allclose(np.asarray(res[key]), t[name].grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=key)


def test_batched_layer_is_per_graph_layer():
    """Graphs of a batch do not see each other: the batched layer's rows of graph b equal
    the layer run on graph b alone."""
    sizes = (5, 12, 7)
    d, heads = 8, 2
    node_ptr, edge_ptr, sl, dl = synth.batch_of_graphs(sizes, 2, np.random.default_rng(4))
    src, dst, _ = oracle.batch_edges(node_ptr, edge_ptr, sl, dl)
    n = int(node_ptr[-1])
    p = synth.gated_layer_inputs(n, d=d)
    whole = oracle.gated_layer(p, oracle.Graph(n, src, dst), heads, node_ptr=node_ptr)
    for b in range(len(sizes)):
        lo, hi = int(node_ptr[b]), int(node_ptr[b + 1])
        pb = dict(p, x=p["x"][lo:hi])
        gb = oracle.Graph(hi - lo, sl[edge_ptr[b]:edge_ptr[b + 1]], dl[edge_ptr[b]:edge_ptr[b + 1]])
        one = oracle.gated_layer(pb, gb, heads)
        np.testing.assert_allclose(whole["out"][lo:hi], one["out"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(whole["S"][b], one["S"], rtol=1e-12, atol=1e-12)
