"""Pins of the oracle's relation-typed messages (GiGL pull request "Support relation message
modes on the packed GraphTransformerEncoder path", section "Approach": per-relation
transforms, mean or softmax weighting, scatter-add, relation edges as packed rows with
host-side (relation, start, end) segments).

- Autograd (library) through a dense formulation: per-relation projections, per-edge
  gathered keys and messages, a [H, N, E] logit matrix masked to each target's in-edges,
  torch.softmax over it (or uniform weights), on multigraphs with several relations between
  the same pair, isolated targets and both weighting modes.
- One relation is plain dot-product local attention (the oracle's own local branch, itself
  pinned against dense attention).
- Mean weighting equals a scatter-mean (numpy add.at and bincount).
- Relabelling the relations (with their transforms) and reordering the edges change
  nothing.
- The segment decoding against a brute-force membership loop, and its rejections.
- The packed-row convention indexes the stacked projection at x_u W^r.
- Central finite differences of the forward for the softmax mode.
"""

import numpy as np
import pytest
import torch

import oracle
import synth


def _case(n, m, n_rel, heads, c, d, seed, isolated=0):
    src, dst = synth.random_multigraph(n, m, seed, self_loops=True, isolated=isolated)
    rng = np.random.default_rng(seed + 100)
    rel = rng.integers(0, n_rel, src.size).astype(np.int32)
    x = rng.standard_normal((n, d))
    w_q = rng.standard_normal((d, heads * c)) * 0.5
    w_k = rng.standard_normal((n_rel, d, heads * c)) * 0.5
    w_v = rng.standard_normal((n_rel, d, heads * c))
    return src, dst, rel, x, w_q, w_k, w_v


def _dense(x, w_q, w_k, w_v, src, dst, rel, n, heads, mean):
    n_rel, _, width = w_v.shape
    c = width // heads
    src_t, dst_t, rel_t = (torch.tensor(a).long() for a in (src, dst, rel))
    keys = torch.stack([x @ w_k[r] for r in range(n_rel)]).reshape(n_rel, n, heads, c)
    vals = torch.stack([x @ w_v[r] for r in range(n_rel)]).reshape(n_rel, n, heads, c)
    k_e, v_e = keys[rel_t, src_t], vals[rel_t, src_t]  # [E, H, C]
    q = (x @ w_q).reshape(n, heads, c)
    s = (q[dst_t] * k_e).sum(-1) * c ** -0.5  # [E, H]
    if mean:
        s = s * 0.0
    member = dst_t[None, :] == torch.arange(n)[:, None]  # [N, E]
    logits = torch.where(member[None], s.T[:, None, :], torch.tensor(-1e30, dtype=s.dtype))
    alpha = torch.softmax(logits, dim=-1) * member[None]  # rows without in-edges -> 0
    out = torch.einsum("hve,ehc->vhc", alpha, v_e)
    return out.reshape(n, heads * c)


@pytest.mark.parametrize("mode", [oracle.REL_SOFTMAX, oracle.REL_MEAN])
@pytest.mark.parametrize("n,m,n_rel,heads,c,seed", [(5, 8, 2, 1, 2, 0), (14, 60, 3, 2, 3, 1), (30, 200, 4, 4, 2, 2)])
def test_relation_matches_dense_autograd(mode, n, m, n_rel, heads, c, seed):
    d = 5
    src, dst, rel, x, w_q, w_k, w_v = _case(n, m, n_rel, heads, c, d, seed, isolated=2)
    d_out = np.random.default_rng(seed + 7).standard_normal((n, heads * c))
    fw = oracle.relation_forward(x, w_q, w_k, w_v, src, dst, rel, heads, mode)
    bw = oracle.relation_backward(x, w_q, w_k, w_v, src, dst, rel, heads, mode, d_out)
    t = [torch.tensor(a).requires_grad_(True) for a in (x, w_q, w_k, w_v)]
    out = _dense(*t, src, dst, rel, n, heads, mode == oracle.REL_MEAN)
    np.testing.assert_allclose(fw["out"], out.detach().numpy(), rtol=1e-12, atol=1e-12)
    (out * torch.tensor(d_out)).sum().backward()
    keys = ("d_x", "d_w_q", "d_w_k", "d_w_v") if mode == oracle.REL_SOFTMAX else ("d_x", "d_w_v")
    for key in keys:
        tt = t[("d_x", "d_w_q", "d_w_k", "d_w_v").index(key)]
        np.testing.assert_allclose(bw[key], tt.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=key)
    if mode == oracle.REL_MEAN:
        assert bw["d_w_q"] is None and bw["d_w_k"] is None
    # isolated targets: no message, log-normaliser -inf
    assert not fw["out"][-2:].any() and np.isneginf(fw["lse"][-2:]).all()


def test_one_relation_is_plain_dot_attention():
    n, heads, c, d = 40, 3, 4, 6
    src, dst, rel, x, w_q, w_k, w_v = _case(n, 300, 1, heads, c, d, 3, isolated=1)
    d_out = np.random.default_rng(3).standard_normal((n, heads, c))
    q, key, val = oracle.relation_projections(x, w_q, w_k, w_v, heads)
    out, lse = oracle.relation_attention(q, key, val, src, dst, rel, oracle.REL_SOFTMAX)
    g = oracle.Graph(n, src, dst)
    o2, l2 = oracle.local_fwd_dot(q, key[0], val[0], g, c ** -0.5)
    np.testing.assert_allclose(out, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, l2, rtol=1e-13, atol=1e-14)
    b = oracle.relation_attention_bwd(q, key, val, d_out, src, dst, rel, oracle.REL_SOFTMAX)
    b2 = oracle.local_bwd_dot(q, key[0], val[0], d_out, g, c ** -0.5)
    np.testing.assert_allclose(b["d_q"], b2["d_q"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(b["d_key"][0], b2["d_k"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(b["d_val"][0], b2["d_v"], rtol=1e-11, atol=1e-13)


def test_mean_is_scatter_mean():
    n, n_rel, heads, c, d = 50, 3, 2, 4, 5
    src, dst, rel, x, _, _, w_v = _case(n, 400, n_rel, heads, c, d, 4, isolated=3)
    out = oracle.relation_forward(x, None, None, w_v, src, dst, rel, heads, oracle.REL_MEAN)
    msg = np.stack([x[src[e]] @ w_v[rel[e]] for e in range(src.size)])
    acc = np.zeros((n, heads * c))
    np.add.at(acc, dst, msg)
    cnt = np.bincount(dst, minlength=n)
    want = acc / np.maximum(cnt, 1)[:, None]
    np.testing.assert_allclose(out["out"], want, rtol=1e-13, atol=1e-14)
    lse_want = np.where(cnt > 0, np.log(np.maximum(cnt, 1)), -np.inf)
    np.testing.assert_allclose(out["lse"], np.repeat(lse_want[:, None], heads, 1), rtol=1e-15)
    # d_x of the mean: each message's transform receives d_out[v] / deg(v)
    d_out = np.random.default_rng(5).standard_normal((n, heads * c))
    b = oracle.relation_backward(x, None, None, w_v, src, dst, rel, heads, oracle.REL_MEAN, d_out)
    g = d_out / np.maximum(cnt, 1)[:, None]
    d_x = np.zeros((n, d))
    for e in range(src.size):
        d_x[src[e]] += g[dst[e]] @ w_v[rel[e]].T
    np.testing.assert_allclose(b["d_x"], d_x, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("mode", [oracle.REL_SOFTMAX, oracle.REL_MEAN])
def test_relabelling_and_edge_order(mode):
    n, n_rel, heads, c, d = 35, 4, 2, 3, 4
    src, dst, rel, x, w_q, w_k, w_v = _case(n, 250, n_rel, heads, c, d, 6)
    base = oracle.relation_forward(x, w_q, w_k, w_v, src, dst, rel, heads, mode)["out"]
    perm = np.array([2, 0, 3, 1])  # relation r becomes perm[r]
    inv = np.argsort(perm)
    relab = oracle.relation_forward(x, w_q, w_k[inv], w_v[inv], src, dst, perm[rel], heads, mode)["out"]
    np.testing.assert_array_equal(relab, base)
    order = np.random.default_rng(6).permutation(src.size)
    shuf = oracle.relation_forward(x, w_q, w_k, w_v, src[order], dst[order], rel[order], heads, mode)["out"]
    np.testing.assert_allclose(shuf, base, rtol=1e-13, atol=1e-14)


def test_segments_decode():
    segs = [(2, 0, 3), (0, 3, 3), (1, 3, 7), (2, 7, 10)]
    rel = oracle.relation_of_segments(10, segs, 3)
    want = []
    for i in range(10):
        want.append([r for r, s, t in segs if s <= i < t][0])
    np.testing.assert_array_equal(rel, want)
    assert oracle.relation_of_segments(0, [], 2).size == 0
    for bad in ([(0, 1, 10)], [(0, 0, 4), (1, 5, 10)], [(0, 0, 4)], [(3, 0, 10)], [(0, 0, 6), (1, 6, 5)],
                [(-1, 0, 10)], [(0, 0, 11)]):
        with pytest.raises(ValueError):
            oracle.relation_of_segments(10, bad, 3)


def test_packed_rows_index_the_stacked_projection():
    n, n_rel, width, d = 9, 3, 4, 5
    rng = np.random.default_rng(7)
    x = rng.standard_normal((n, d))
    w = rng.standard_normal((n_rel, d, width))
    stacked = (x @ np.concatenate(list(w), axis=1)).reshape(n * n_rel, width)
    src = np.array([0, 8, 4, 9, -1, 3], np.int32)
    rel = np.array([0, 2, 1, 0, 1, 2], np.int32)
    rows, bad = oracle.relation_rows(src, rel, n, n_rel)
    assert bad == 2 and rows[3] == -1 and rows[4] == -1
    for e in (0, 1, 2, 5):
        np.testing.assert_allclose(stacked[rows[e]], x[src[e]] @ w[rel[e]], rtol=1e-14)


def test_relation_finite_differences():
    n, n_rel, heads, c, d = 8, 2, 2, 2, 3
    src, dst, rel, x, w_q, w_k, w_v = _case(n, 25, n_rel, heads, c, d, 8)
    d_out = np.random.default_rng(8).standard_normal((n, heads * c))
    b = oracle.relation_backward(x, w_q, w_k, w_v, src, dst, rel, heads, oracle.REL_SOFTMAX, d_out)

    def loss(**kw):
        a = dict(x=x, w_q=w_q, w_k=w_k, w_v=w_v)
        a.update(kw)
        out = oracle.relation_forward(a["x"], a["w_q"], a["w_k"], a["w_v"], src, dst, rel, heads,
                                      oracle.REL_SOFTMAX)["out"]
        return float((out * d_out).sum())

    h = 1e-6
    for name, arr, idx in (("x", x, (3, 1)), ("w_q", w_q, (2, 3)), ("w_k", w_k, (1, 0, 2)), ("w_v", w_v, (0, 2, 1))):
        p, m = arr.copy(), arr.copy()
        p[idx] += h
        m[idx] -= h
        fd = (loss(**{name: p}) - loss(**{name: m})) / (2 * h)
        assert abs(fd - b["d_" + name][idx]) < 1e-7 * max(1.0, abs(fd)), name
