"""Pins of the oracle's dot-product local attention (forward and backward).

What fixes the result, independent of the oracle's own loops:
- torch's scaled_dot_product_attention (a library routine) in float64 on the dense
  N x N score matrix, masked to the graph: the local branch L_i of "Gated
  Local-Global Graph Attention" (Key formulas) is exactly masked softmax attention.
  Duplicate edges enter as multiplicity weights, i.e. an additive log(count) mask.
- On the complete graph the local branch is dense multi-head attention
  (ag_multihead_attention, Details: per-head softmax of q_h^T k_h / sqrt(d_k)).
- Autograd through that library routine pins the backward; central finite
  differences of the oracle's forward pin it a second way.
- Invariants: weights sum to one per non-empty row, a self-loop-only row returns its
  own value row, results do not depend on COO order, vertex labels or head order, and
  huge scores stay finite (Tinymesh "Evidence and limits").
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _dense_mask(n, src, dst):
    cnt = np.zeros((n, n))
    np.add.at(cnt, (dst, src), 1.0)
    with np.errstate(divide="ignore"):
        return np.log(cnt), cnt  # -inf where no edge


def _sdpa(q, k, v, mask, scale):
    # [N,H,C] -> [H,N,C]
    tq, tk, tv = (torch.tensor(a).permute(1, 0, 2).contiguous() for a in (q, k, v))
    m = torch.tensor(mask)
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale)
    return out.permute(1, 0, 2).numpy()


GRAPHS = [
    # n, m, seed, self_loops, isolated
    (1, 0, 0, True, 0),
    (2, 3, 1, True, 0),
    (12, 40, 2, True, 0),
    (33, 200, 3, True, 3),
    (64, 600, 4, False, 5),
    (64, 4000, 5, True, 0),
]


@pytest.mark.parametrize("n,m,seed,loops,iso", GRAPHS)
@pytest.mark.parametrize("hh,c", [(1, 4), (3, 5)])
def test_dot_fwd_matches_masked_sdpa(n, m, seed, loops, iso, hh, c):
    src, dst = synth.random_multigraph(n, m, seed, self_loops=loops, isolated=iso)
    g = oracle.Graph(n, src, dst)
    q, k, v = _rand((n, hh, c), seed), _rand((n, hh, c), seed + 100), _rand((n, hh, c), seed + 200)
    scale = 1.0 / np.sqrt(c)
    out, lse = oracle.local_fwd_dot(q, k, v, g, scale)
    logm, cnt = _dense_mask(n, src, dst)
    live = cnt.sum(1) > 0
    if live.any():
        ref = _sdpa(q, k, v, logm, scale)
        np.testing.assert_allclose(out[live], ref[live], rtol=1e-12, atol=1e-12)
        # lse against a library logsumexp of the masked scores
        s = np.einsum("vhc,uhc->hvu", q, k) * scale + logm[None]
        ref_lse = torch.logsumexp(torch.tensor(s), dim=-1).numpy().T
        np.testing.assert_allclose(lse[live], ref_lse[live], rtol=1e-12, atol=1e-12)
    # rows with no in-edge: zero output and lse = -inf, never NaN
    assert np.all(out[~live] == 0.0)
    assert np.all(np.isneginf(lse[~live]))


def test_complete_graph_is_dense_mha():
    n, hh, c = 20, 4, 8
    u, v = np.meshgrid(np.arange(n), np.arange(n))
    src, dst = u.ravel().astype(np.int32), v.ravel().astype(np.int32)
    g = oracle.Graph(n, src, dst)
    q, k, vv = _rand((n, hh, c), 1), _rand((n, hh, c), 2), _rand((n, hh, c), 3)
    out, _ = oracle.local_fwd_dot(q, k, vv, g, 1.0 / np.sqrt(c))
    tq, tk, tv = (torch.tensor(a).permute(1, 0, 2) for a in (q, k, vv))
    ref = F.scaled_dot_product_attention(tq, tk, tv).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_weights_sum_to_one_and_self_loop_row():
    n, hh, c = 30, 2, 3
    src, dst = synth.random_multigraph(n, 100, 7, self_loops=True, isolated=4)
    # node n-1 is isolated by the generator; give node n-2 ... keep as is and add a lone self-loop node
    src = np.concatenate([src, [n]]).astype(np.int32)
    dst = np.concatenate([dst, [n]]).astype(np.int32)
    n += 1
    g = oracle.Graph(n, src, dst)
    q, k = _rand((n, hh, c), 1) * 3, _rand((n, hh, c), 2) * 3
    ones = np.ones((n, hh, c))
    out, _ = oracle.local_fwd_dot(q, k, ones, g, 0.7)
    deg = np.diff(g.row_ptr)
    np.testing.assert_allclose(out[deg > 0], 1.0, rtol=0, atol=1e-14)
    v = _rand((n, hh, c), 3)
    out, lse = oracle.local_fwd_dot(q, k, v, g, 0.7)
    np.testing.assert_array_equal(out[n - 1], v[n - 1])
    np.testing.assert_allclose(lse[n - 1], 0.7 * (q[n - 1] * k[n - 1]).sum(-1), rtol=1e-14)


def test_invariance_coo_order_vertex_labels_heads():
    n, hh, c = 40, 3, 4
    src, dst = synth.random_multigraph(n, 300, 8, self_loops=True, isolated=2)
    q, k, v = _rand((n, hh, c), 4), _rand((n, hh, c), 5), _rand((n, hh, c), 6)
    base, base_lse = oracle.local_fwd_dot(q, k, v, oracle.Graph(n, src, dst), 0.5)
    rng = np.random.default_rng(9)
    p = rng.permutation(src.size)
    out, _ = oracle.local_fwd_dot(q, k, v, oracle.Graph(n, src[p], dst[p]), 0.5)
    np.testing.assert_allclose(out, base, rtol=1e-13, atol=1e-14)
    relabel = rng.permutation(n).astype(np.int32)  # old id -> new id
    inv = np.argsort(relabel)
    g2 = oracle.Graph(n, relabel[src], relabel[dst])
    out2, lse2 = oracle.local_fwd_dot(q[inv], k[inv], v[inv], g2, 0.5)
    np.testing.assert_allclose(out2[relabel], base, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2[relabel], base_lse, rtol=1e-13, atol=1e-14)
    hp = np.array([2, 0, 1])
    out3, _ = oracle.local_fwd_dot(q[:, hp], k[:, hp], v[:, hp], oracle.Graph(n, src, dst), 0.5)
    np.testing.assert_array_equal(out3, base[:, hp])


def test_large_scores_stay_finite():
    n, hh, c = 16, 2, 4
    src, dst = synth.random_multigraph(n, 60, 10, self_loops=True)
    q, k, v = _rand((n, hh, c), 1) * 100.0, _rand((n, hh, c), 2) * 100.0, _rand((n, hh, c), 3)
    g = oracle.Graph(n, src, dst)
    out, lse = oracle.local_fwd_dot(q, k, v, g, 1.0)  # scores of order 1e4
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    logm, _ = _dense_mask(n, src, dst)
    np.testing.assert_allclose(out, _sdpa(q, k, v, logm, 1.0), rtol=1e-10, atol=1e-10)


def test_row_subset_matches_full():
    n = 50
    src, dst = synth.random_multigraph(n, 400, 12, isolated=3)
    g = oracle.Graph(n, src, dst)
    q, k, v = _rand((n, 2, 3), 1), _rand((n, 2, 3), 2), _rand((n, 2, 3), 3)
    full, full_lse = oracle.local_fwd_dot(q, k, v, g, 0.3)
    rows = np.array([49, 0, 7, 7, 22], np.int32)
    sub, sub_lse = oracle.local_fwd_dot(q, k, v, g, 0.3, rows=rows)
    np.testing.assert_array_equal(sub, full[rows])
    np.testing.assert_array_equal(sub_lse, full_lse[rows])


# --------------------------------------------------------------------------- backward


@pytest.mark.parametrize("n,m,seed,iso", [(2, 2, 0, 0), (12, 40, 1, 0), (40, 300, 2, 4), (64, 2000, 3, 0)])
def test_dot_bwd_matches_autograd(n, m, seed, iso):
    hh, c = 2, 3
    src, dst = synth.random_multigraph(n, m, seed, self_loops=True, isolated=iso)
    g = oracle.Graph(n, src, dst)
    q, k, v = _rand((n, hh, c), seed), _rand((n, hh, c), seed + 1), _rand((n, hh, c), seed + 2)
    d_out = _rand((n, hh, c), seed + 3)
    scale = 1.0 / np.sqrt(c)
    r = oracle.local_bwd_dot(q, k, v, d_out, g, scale)
    logm, cnt = _dense_mask(n, src, dst)
    live = cnt.sum(1) > 0
    # isolated destinations: the library routine would give NaN rows; give them a dummy
    # key so the mask is finite, and zero their upstream gradient.
    m_safe = logm.copy()
    m_safe[~live, 0] = 0.0
    dO = d_out.copy()
    dO[~live] = 0.0
    tq, tk, tv = (torch.tensor(a).permute(1, 0, 2).contiguous().requires_grad_(True) for a in (q, k, v))
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(m_safe), scale=scale)
    (out * torch.tensor(dO).permute(1, 0, 2)).sum().backward()
    for name, t in (("d_q", tq), ("d_k", tk), ("d_v", tv)):
        np.testing.assert_allclose(r[name], t.grad.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12, err_msg=name)
    # D = sum alpha * d alpha equals d_out . out per head (closed form)
    fwd, _ = oracle.local_fwd_dot(q, k, v, g, scale)
    np.testing.assert_allclose(r["D"][live], (d_out * fwd).sum(-1)[live], rtol=1e-11, atol=1e-12)
    assert np.all(r["d_q"][~live] == 0.0)


def test_dot_bwd_finite_differences():
    n, hh, c = 9, 2, 3
    src, dst = synth.random_multigraph(n, 25, 21, self_loops=True, isolated=1)
    g = oracle.Graph(n, src, dst)
    q, k, v = _rand((n, hh, c), 31), _rand((n, hh, c), 32), _rand((n, hh, c), 33)
    d_out = _rand((n, hh, c), 34)
    scale = 0.6
    r = oracle.local_bwd_dot(q, k, v, d_out, g, scale)

    def loss(qq, kk, vv):
        o, _ = oracle.local_fwd_dot(qq, kk, vv, g, scale)
        return float((o * d_out).sum())

    h = 1e-6
    for which, grad in ((0, r["d_q"]), (1, r["d_k"]), (2, r["d_v"])):
        for idx in np.ndindex(n, hh, c):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            lp = loss(*args)
            args[which][idx] -= 2 * h
            lm = loss(*args)
            assert abs((lp - lm) / (2 * h) - grad[idx]) < 1e-7, (which, idx)


def test_dot_bwd_row_subsets():
    n, hh, c = 30, 2, 2
    src, dst = synth.random_multigraph(n, 150, 41, self_loops=True, isolated=2)
    g = oracle.Graph(n, src, dst)
    q, k, v, d = (_rand((n, hh, c), s) for s in (1, 2, 3, 4))
    full = oracle.local_bwd_dot(q, k, v, d, g, 0.5)
    rd = np.array([3, 29, 0], np.int32)
    rs = np.array([5, 5, 28], np.int32)
    sub = oracle.local_bwd_dot(q, k, v, d, g, 0.5, rows_d=rd, rows_s=rs)
    np.testing.assert_array_equal(sub["d_q"], full["d_q"][rd])
    np.testing.assert_array_equal(sub["d_k"], full["d_k"][rs])
    np.testing.assert_array_equal(sub["d_v"], full["d_v"][rs])
