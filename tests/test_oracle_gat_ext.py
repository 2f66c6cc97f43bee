"""Pins of the oracle's GAT variants the Tinymesh page lists as not yet covered (section
"Evidence and limits"): head averaging and learned edge features in the score, read as in
the GATConv its "Reference contract" section follows (an edge term a_e . (F W_e) added to the
logit before LeakyReLU; concat=False averages the heads).

- Autograd (library) through a dense edge-wise formulation: a [K, N, E] logit matrix masked
  to each target's in-edges, torch.softmax over it, on multigraphs (duplicate edges carry
  their own features), both concatenated and averaged heads.
- Where every edge has its own source, the edge term is exactly a shift of that source's
  coefficient: the oracle with the term equals the oracle without it on shifted s_src,
  and d s_edge equals the plain path's d s_src.
- Zero edge attention reproduces the plain layer bit for bit.
- Central finite differences of the local forward for d s_edge.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


def _dense_edge_gat(x, w, a_s, a_t, f, w_e, a_e, src, dst, n, slope, concat):
    heads, c = a_s.shape
    e = len(src)
    hf = (x @ w).reshape(n, heads, c)
    s_src = (hf * a_s[None]).sum(-1)
    s_dst = (hf * a_t[None]).sum(-1)
    he = (f @ w_e).reshape(e, heads, c)
    s_edge = (he * a_e[None]).sum(-1)  # [E, K]
    src_t, dst_t = torch.tensor(src).long(), torch.tensor(dst).long()
    z = F.leaky_relu(s_src[src_t] + s_dst[dst_t] + s_edge, slope)  # [E, K]
    member = dst_t[None, :] == torch.arange(n)[:, None]  # [N, E]
    logits = torch.where(member[None], z.T[:, None, :], torch.tensor(-torch.inf, dtype=z.dtype))
    alpha = torch.softmax(logits, dim=-1)  # [K, N, E]
    out = torch.einsum("kve,ekc->vkc", alpha, hf[src_t])
    return out.reshape(n, heads * c) if concat else out.mean(1)


@pytest.mark.parametrize("concat", [True, False])
@pytest.mark.parametrize("n,m,seed,heads,c,fe", [(4, 6, 0, 1, 2, 3), (12, 50, 1, 2, 3, 4), (25, 160, 2, 4, 2, 5)])
def test_edge_gat_matches_dense_autograd(concat, n, m, seed, heads, c, fe):
    src, dst = synth.random_multigraph(n, m, seed, self_loops=True)
    g = oracle.Graph(n, src, dst)
    e = len(src)
    rng = np.random.default_rng(seed + 10)
    fin = 5
    x = rng.standard_normal((n, fin))
    w = rng.standard_normal((fin, heads * c)) * 0.5
    a_s, a_t, a_e = (rng.standard_normal((heads, c)) for _ in range(3))
    fe_x = rng.standard_normal((e, fe))
    w_e = rng.standard_normal((fe, heads * c)) * 0.5
    d_out = rng.standard_normal((n, heads * c if concat else c))
    edge = dict(f=fe_x, w_e=w_e, a_e=a_e)
    fw = oracle.gat_forward(x, w, a_s, a_t, g, concat=concat, edge=edge)
    bw = oracle.gat_backward(x, w, a_s, a_t, d_out, g, concat=concat, edge=edge)
    t = [torch.tensor(a).requires_grad_(True) for a in (x, w, a_s, a_t, fe_x, w_e, a_e)]
    out = _dense_edge_gat(*t, src, dst, n, oracle.SLOPE, concat)
    np.testing.assert_allclose(fw["out"], out.detach().numpy(), rtol=1e-12, atol=1e-12)
    (out * torch.tensor(d_out)).sum().backward()
    for key, tt in zip(("d_x", "d_w", "d_a_s", "d_a_t", "d_f", "d_w_e", "d_a_e"), t):
        np.testing.assert_allclose(bw[key], tt.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=key)


def test_edge_term_is_a_source_shift_when_sources_are_unique():
    n, heads, c = 40, 3, 4
    rng = np.random.default_rng(4)
    src = rng.permutation(n).astype(np.int32)  # every node sends exactly one edge
    dst = rng.integers(0, n, n).astype(np.int32)
    g = oracle.Graph(n, src, dst)
    s_src, s_dst = rng.standard_normal((n, heads)), rng.standard_normal((n, heads))
    s_edge = rng.standard_normal((n, heads))
    hf = rng.standard_normal((n, heads, c))
    d_out = rng.standard_normal((n, heads, c))
    shifted = s_src.copy()
    shifted[src] += s_edge
    out, lse = oracle.local_fwd_add(s_src, s_dst, hf, g, s_edge=s_edge)
    out2, lse2 = oracle.local_fwd_add(shifted, s_dst, hf, g)
    np.testing.assert_allclose(out, out2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse, lse2, rtol=1e-14)
    b = oracle.local_bwd_add(s_src, s_dst, hf, d_out, g, s_edge=s_edge)
    b2 = oracle.local_bwd_add(shifted, s_dst, hf, d_out, g)
    np.testing.assert_allclose(b["d_s_edge"], b2["d_s_src"][src], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(b["d_s_dst"], b2["d_s_dst"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(b["d_hf"], b2["d_hf"], rtol=1e-13, atol=1e-15)


def test_zero_edge_attention_is_the_plain_layer():
    n, heads, c = 30, 2, 3
    src, dst = synth.random_multigraph(n, 150, 6, self_loops=True, isolated=2)
    g = oracle.Graph(n, src, dst)
    rng = np.random.default_rng(6)
    x, w = rng.standard_normal((n, 4)), rng.standard_normal((4, heads * c))
    a_s, a_t = rng.standard_normal((heads, c)), rng.standard_normal((heads, c))
    edge = dict(f=rng.standard_normal((len(src), 3)), w_e=rng.standard_normal((3, heads * c)),
                a_e=np.zeros((heads, c)))
    d_out = rng.standard_normal((n, heads * c))
    plain = oracle.gat_forward(x, w, a_s, a_t, g)
    with_e = oracle.gat_forward(x, w, a_s, a_t, g, edge=edge)
    np.testing.assert_array_equal(with_e["out"], plain["out"])
    bp = oracle.gat_backward(x, w, a_s, a_t, d_out, g)
    be = oracle.gat_backward(x, w, a_s, a_t, d_out, g, edge=edge)
    for key in ("d_x", "d_w", "d_a_s", "d_a_t"):
        np.testing.assert_array_equal(be[key], bp[key])
    assert not be["d_w_e"].any() and not be["d_f"].any()


def test_head_average_is_the_mean_of_the_heads():
    n, heads, c = 20, 4, 3
    src, dst = synth.random_multigraph(n, 90, 7, self_loops=True)
    g = oracle.Graph(n, src, dst)
    rng = np.random.default_rng(7)
    x, w = rng.standard_normal((n, 5)), rng.standard_normal((5, heads * c))
    a_s, a_t = rng.standard_normal((heads, c)), rng.standard_normal((heads, c))
    cat = oracle.gat_forward(x, w, a_s, a_t, g)["out"].reshape(n, heads, c)
    avg = oracle.gat_forward(x, w, a_s, a_t, g, concat=False)["out"]
    np.testing.assert_allclose(avg, cat.mean(1), rtol=1e-15, atol=1e-15)


def test_edge_gradient_finite_differences():
    n, heads, c = 10, 2, 2
    src, dst = synth.random_multigraph(n, 30, 8, self_loops=True)
    g = oracle.Graph(n, src, dst)
    rng = np.random.default_rng(8)
    s_src, s_dst = rng.standard_normal((n, heads)), rng.standard_normal((n, heads))
    s_edge = rng.standard_normal((len(src), heads))
    hf = rng.standard_normal((n, heads, c))
    d_out = rng.standard_normal((n, heads, c))
    b = oracle.local_bwd_add(s_src, s_dst, hf, d_out, g, s_edge=s_edge)

    def loss(se):
        return float((oracle.local_fwd_add(s_src, s_dst, hf, g, s_edge=se)[0] * d_out).sum())

    h = 1e-6
    for e_i in (0, 7, len(src) - 1):
        for k in range(heads):
            sp, sm = s_edge.copy(), s_edge.copy()
            sp[e_i, k] += h
            sm[e_i, k] -= h
            z = s_src[src[e_i], k] + s_dst[dst[e_i], k] + s_edge[e_i, k]
            if abs(z) < 1e-3:  # the LeakyReLU kink
                continue
            assert abs((loss(sp) - loss(sm)) / (2 * h) - b["d_s_edge"][e_i, k]) < 1e-7


def test_coefficients_select_columns_for_identity_weights():
    """Closed-form special case of both coefficient maps: with W = I and a one-hot attention
    vector per head (entry j_k of head k), the coefficient of row n and head k is the input's
    column k*C + j_k (Tinymesh "Composition": one coefficient per node and head of X W)."""
    rng = np.random.default_rng(3)
    n, heads, c = 7, 3, 4
    x = rng.standard_normal((n, heads * c))
    j = np.array([2, 0, 3])
    a = np.zeros((heads, c))
    a[np.arange(heads), j] = 1.0
    b = np.zeros((heads, c))
    b[np.arange(heads), (j + 1) % c] = 1.0
    hf, s_src, s_dst = oracle.gat_coefficients(x, np.eye(heads * c), a, b)
    np.testing.assert_array_equal(hf.reshape(n, -1), x)
    np.testing.assert_array_equal(s_src, x[:, np.arange(heads) * c + j])
    np.testing.assert_array_equal(s_dst, x[:, np.arange(heads) * c + (j + 1) % c])
    he, s_edge = oracle.edge_coefficients(x, np.eye(heads * c), a)
    np.testing.assert_array_equal(he.reshape(n, -1), x)
    np.testing.assert_array_equal(s_edge, x[:, np.arange(heads) * c + j])


def test_coefficients_follow_a_head_permutation():
    """Permuting the heads (W's column blocks with the rows of a_s, a_t) permutes the
    coefficients' head axis the same way."""
    rng = np.random.default_rng(4)
    n, fin, heads, c = 9, 5, 4, 3
    x, w = rng.standard_normal((n, fin)), rng.standard_normal((fin, heads * c))
    a_s, a_t = rng.standard_normal((heads, c)), rng.standard_normal((heads, c))
    perm = np.array([2, 0, 3, 1])
    wp = w.reshape(fin, heads, c)[:, perm].reshape(fin, heads * c)
    _, s1, d1 = oracle.gat_coefficients(x, w, a_s, a_t)
    _, s2, d2 = oracle.gat_coefficients(x, wp, a_s[perm], a_t[perm])
    np.testing.assert_allclose(s2, s1[:, perm], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(d2, d1[:, perm], rtol=1e-12, atol=1e-12)


def test_phi_grad_matches_finite_differences():
    """d phi / dx (phi = elu + 1) against central differences of the oracle's phi, away from
    the kink at 0 where the one-sided derivatives (1 and e^0 = 1) agree anyway."""
    x = np.concatenate([np.linspace(-6, -0.01, 50), np.linspace(0.01, 6, 50)])
    h = 1e-6
    fd = (oracle.phi(x + h) - oracle.phi(x - h)) / (2 * h)
    np.testing.assert_allclose(oracle.phi_grad(x), fd, rtol=1e-7, atol=1e-8)
    assert oracle.phi_grad(np.array([0.0]))[0] == 1.0
