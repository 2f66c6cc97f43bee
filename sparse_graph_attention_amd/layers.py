"""The two layers the pages build from the primitives, as sequences of libgga calls.

Nothing here computes: each function only orders entry points of the C ABI and hands
tensors from one to the next.

- GAT layer (Tinymesh "Sparse attention experiment", sections "Composition" and
  "Multiple heads are composition"): H = X W, per-node coefficients, additive scores,
  target softmax, weighted sum, heads concatenated; and its first-order gradients.
- Gated local-global layer ("Gated Local-Global Graph Attention", Implementation notes
  item 2): Q, K, V projections, local masked softmax, phi = elu+1 global branch, node
  gate, W_o, residual LayerNorm.
- Relation-typed messages (GiGL pull request "Support relation message modes on the
  packed GraphTransformerEncoder path", section "Approach"): per-relation key and message
  transforms of every node, relation edges mapped to (node, relation) rows, then softmax
  or mean weighting over each target's in-edges and the weighted sum.
"""

from __future__ import annotations

import torch

from . import (GGA_BF16, GGA_F32, GGA_SCORE_ADDITIVE, GGA_SCORE_DOT, GGA_SCORE_MEAN, Topology, gga_add_layernorm,
               gga_add_layernorm_bwd, gga_gat_coef_bwd, gga_gat_coef_fwd, gga_gated_combine, gga_gated_combine_bwd,
               gga_head_mean, gga_head_mean_bwd, gga_local_attn_bwd_edge, gga_local_attn_fwd_edge,
               gga_qkv_gate_proj, gga_qkv_proj_bwd_x,
               gga_global_linear_batch_bwd, gga_global_linear_batch_fwd, gga_global_linear_bwd,
               gga_global_linear_fwd, gga_linear, gga_linear_accumulate, gga_local_attn_bwd, gga_local_attn_fwd,
               gga_relation_sources, make_desc)


def gat_forward(x: torch.Tensor, w: torch.Tensor, a_s: torch.Tensor, a_t: torch.Tensor, topo: Topology,
                negative_slope: float = 0.2, concat: bool = True, edge: dict | None = None):
    """Returns a dict with out (heads concatenated [N, K*C], or averaged [N, C] with
    concat=False) and the intermediates the backward needs.  edge = dict(f [E, Fe] in COO
    order, w_e [Fe, K*C], a_e [K, C]) adds the learned edge term a_e . (F W_e) to every
    logit."""
    n = x.shape[0]
    heads, c = a_s.shape
    hf = gga_linear(x, w).view(n, heads, c)
    s_src, s_dst = gga_gat_coef_fwd(hf, a_s, a_t)
    desc = make_desc(n, topo.e, heads, c, GGA_SCORE_ADDITIVE, GGA_F32, 1.0, negative_slope)
    g_e = s_edge = None
    if edge is None:
        out, lse = gga_local_attn_fwd(desc, s_dst, s_src, hf, topo.row_ptr, topo.col, topo.plan)
    else:
        # s_edge[e,k] = a_e[k] . (F W_e)[e,k] = F[e] . G[:,k] with G[f,k] = a_e[k] . W_e[f,k]:
        # the [E, K*C] edge state is never formed
        fe = edge["f"].shape[1]
        g_e, _ = gga_gat_coef_fwd(edge["w_e"].view(fe, heads, c), edge["a_e"], None)
        s_edge = gga_linear(edge["f"], g_e)
        out, lse = gga_local_attn_fwd_edge(desc, s_dst, s_src, hf, s_edge, topo)
    res = out.view(n, heads * c) if concat else gga_head_mean(out)
    return dict(out=res, hf=hf, s_src=s_src, s_dst=s_dst, lse=lse, desc=desc, out3=out, g_e=g_e, s_edge=s_edge)


def gat_backward(x, w, a_s, a_t, d_out: torch.Tensor, fwd: dict, topo: Topology, concat: bool = True,
                 edge: dict | None = None):
    """dX, dW, da_s, da_t (and with edge features dF, dW_e, da_e) of sum(out * d_out)
    (Tinymesh "Evidence and limits": first-order gradients).  topo must hold the CSR by
    source (Topology(..., backward=True))."""
    n = x.shape[0]
    heads, c = a_s.shape
    d3 = d_out.reshape(n, heads, c) if concat else gga_head_mean_bwd(d_out, heads)
    res = {}
    if edge is None:
        d_sdst, d_ssrc, d_hf_attn = gga_local_attn_bwd(fwd["desc"], fwd["s_dst"], fwd["s_src"], fwd["hf"],
                                                       fwd["out3"], fwd["lse"], d3, topo)
    else:
        d_sdst, d_ssrc, d_hf_attn, d_se = gga_local_attn_bwd_edge(fwd["desc"], fwd["s_dst"], fwd["s_src"], fwd["hf"],
                                                                  fwd["s_edge"], fwd["out3"], fwd["lse"], d3, topo)
        # dG = F^T d s_edge, dF = d s_edge G^T; through G[f,k] = a_e[k] . W_e[f,k]:
        # dW_e[f,k,:] = dG[f,k] a_e[k] and da_e[k,:] = sum_f dG[f,k] W_e[f,k,:]
        fe = edge["f"].shape[1]
        d_g = gga_linear(edge["f"], d_se, trans_a=True)
        d_w_e, d_a_e, _ = gga_gat_coef_bwd(edge["w_e"].view(fe, heads, c), edge["a_e"], None, None, d_g, None)
        res.update(d_s_edge=d_se, d_a_e=d_a_e, d_w_e=d_w_e.view(fe, heads * c),
                   d_f=gga_linear(d_se, fwd["g_e"], trans_b=True))
    d_hf, d_a_s, d_a_t = gga_gat_coef_bwd(fwd["hf"], a_s, a_t, d_hf_attn, d_ssrc, d_sdst)
    dh = d_hf.view(n, heads * c)
    d_w = gga_linear(x, dh, trans_a=True)
    d_x = gga_linear(dh, w, trans_b=True)
    res.update(d_x=d_x, d_w=d_w, d_a_s=d_a_s, d_a_t=d_a_t, d_hf=d_hf, d_s_src=d_ssrc, d_s_dst=d_sdst)
    return res


def gated_layer_forward(p: dict, topo: Topology, heads: int, eps: float = 1e-6, ln_eps: float = 1e-5,
                        dtype: int = GGA_F32, node_ptr: torch.Tensor | None = None):
    """p: x [N,d], w_q, w_k, w_v, w_o [d,d], w_g [d], b_g (float), gamma, beta [d].
    node_ptr (int32 [B+1], device): the rows are a batch of B graphs packed along the node
    axis, topo their block-diagonal union (gga_batch_edges); the global statistics are
    then per graph."""
    x = p["x"]
    n, d = x.shape
    r = d // heads
    # [Q | K | V | gate logit] = X [W_Q | W_K | W_V | w_g] + [0 | 0 | 0 | b_g], X read once
    q, k, v, logit = gga_qkv_gate_proj(x, p["w_q"], p["w_k"], p["w_v"], p["w_g"], p["b_g"], heads)
    desc = make_desc(n, topo.e, heads, r, GGA_SCORE_DOT, dtype, r ** -0.5)
    loc, lse = gga_local_attn_fwd(desc, q, k, v, topo.row_ptr, topo.col, topo.plan)
    if node_ptr is None:
        s, z, glob = gga_global_linear_fwd(q, k, v, eps)
    else:
        s, z, glob = gga_global_linear_batch_fwd(node_ptr, q, k, v, eps)
    gate, y = gga_gated_combine(logit, loc.view(n, d), glob.view(n, d))
    zo = gga_linear(y, p["w_o"])
    out = gga_add_layernorm(x, zo, p["gamma"], p["beta"], ln_eps)
    return dict(q=q, k=k, v=v, local=loc.view(n, d), local3=loc, lse=lse, S=s, z=z, glob=glob.view(n, d), gate=gate,
                y=y, zo=zo, out=out, desc=desc)


def gated_layer_backward(p: dict, fwd: dict, topo: Topology, heads: int, d_out: torch.Tensor, eps: float = 1e-6,
                         ln_eps: float = 1e-5, node_ptr: torch.Tensor | None = None, mark=None):
    """First-order gradients of sum(out * d_out) for every input and parameter of the gated
    local-global layer, from the forward's intermediates.  topo must hold the CSR by source
    (Topology(..., backward=True)); the forward must have run in fp32.  mark (optional) is
    called with "local_bwd0" and "local_bwd1" on the host right before and after the local
    attention's backward call is enqueued (a benchmark records stream events there)."""
    x = p["x"]
    n, d = x.shape
    r = d // heads
    d_pre, d_gamma, d_beta = gga_add_layernorm_bwd(x, fwd["zo"], p["gamma"], d_out, ln_eps)
    d_y = gga_linear(d_pre, p["w_o"], trans_b=True)
    d_wo = gga_linear(fwd["y"], d_pre, trans_a=True)
    # the gate logit's share of dX (d_logit w_g^T) is added by the dX product below, into
    # d_pre, the residual's share; the combine backward does not read or write an [n, d]
    # gradient for it
    d_loc, d_glob, _, d_wg, d_bg, d_logit = gga_gated_combine_bwd(x, p["w_g"], p["b_g"], fwd["local"], fwd["glob"],
                                                                  d_y, None)
    d_x = d_pre
    if mark is not None:
        mark("local_bwd0")
    d_q, d_k, d_v = gga_local_attn_bwd(fwd["desc"], fwd["q"], fwd["k"], fwd["v"], fwd["local3"], fwd["lse"],
                                       d_loc.view(n, heads, r), topo)
    if mark is not None:
        mark("local_bwd1")
    if node_ptr is None:
        gga_global_linear_bwd(fwd["q"], fwd["k"], fwd["v"], fwd["S"], fwd["z"], d_glob.view(n, heads, r), d_q, d_k,
                              d_v, eps, g_fw=fwd["glob"].view(n, heads, r))
    else:
        gga_global_linear_batch_bwd(node_ptr, fwd["q"], fwd["k"], fwd["v"], fwd["S"], fwd["z"],
                                    d_glob.view(n, heads, r), d_q, d_k, d_v, eps, g_fw=fwd["glob"].view(n, heads, r))
    grads = dict(d_w_o=d_wo, d_w_g=d_wg, d_b_g=d_bg, d_gamma=d_gamma, d_beta=d_beta)
    for name, g in (("q", d_q), ("k", d_k), ("v", d_v)):
        grads["d_w_" + name] = gga_linear(x, g.view(n, d), trans_a=True)
    # d_x += [dQ | dK | dV] [W_Q | W_K | W_V]^T + d_logit w_g^T in one product
    gga_qkv_proj_bwd_x(d_q, d_k, d_v, p["w_q"], p["w_k"], p["w_v"], d_x, d_logit=d_logit, w_g=p["w_g"])
    grads["d_x"] = d_x
    return grads


def relation_topology(n: int, n_rel: int, src: torch.Tensor, dst: torch.Tensor, segments, backward: bool = False):
    """Relation edges as packed rows (src, dst) grouped by relation, with host-side
    (relation, start, end) segments: each source becomes its (node, relation) row
    u * R + r and the topology is built over n targets and n * R source rows.  Returns
    (topology, d_bad); d_bad (device int32) counts endpoints outside [0, n), and no
    attention call may run on the topology unless it is 0."""
    src_rel, bad = gga_relation_sources(n, n_rel, src, dst, segments)
    return Topology(n, src_rel, dst, backward=backward, n_src=n * n_rel), bad


def relation_forward(x: torch.Tensor, w_q, w_k, w_v: torch.Tensor, topo: Topology, heads: int, n_rel: int,
                     mean: bool):
    """Relation-typed messages.  x [N, d]; w_k, w_v [d, R*W] hold the R relation transforms
    side by side (columns r*W .. r*W+W-1 are W^r), so that X w_v viewed as [N*R, W] has the
    message of node u under relation r in row u*R + r; w_q [d, W].  Softmax mode: per head,
    softmax over v's in-edges of q_v . k_{u,r} / sqrt(C); mean mode (w_q, w_k unused): each
    in-edge weighs 1/deg(v).  topo from relation_topology.  Returns out [N, W] and the
    intermediates the backward needs."""
    n = x.shape[0]
    width = w_v.shape[1] // n_rel
    c = width // heads
    v = gga_linear(x, w_v).view(n * n_rel, heads, c)
    if mean:
        desc = make_desc(n, topo.e, heads, c, GGA_SCORE_MEAN, GGA_F32, 1.0, n_src=n * n_rel)
        q = k = None
    else:
        desc = make_desc(n, topo.e, heads, c, GGA_SCORE_DOT, GGA_F32, c ** -0.5, n_src=n * n_rel)
        q = gga_linear(x, w_q).view(n, heads, c)
        k = gga_linear(x, w_k).view(n * n_rel, heads, c)
    out, lse = gga_local_attn_fwd(desc, q, k, v, topo.row_ptr, topo.col, topo.plan, want_lse=not mean)
    return dict(out=out.view(n, width), out3=out, lse=lse, q=q, k=k, v=v, desc=desc)


def relation_backward(x: torch.Tensor, w_q, w_k, w_v: torch.Tensor, d_out: torch.Tensor, fwd: dict, topo: Topology,
                      heads: int, n_rel: int, mean: bool):
    """dX, dW_V (and in softmax mode dW_Q, dW_K) of sum(out * d_out), in the layouts of
    relation_forward.  topo must hold the CSR by source (relation_topology(...,
    backward=True))."""
    n = x.shape[0]
    width = w_v.shape[1] // n_rel
    c = width // heads
    d3 = d_out.reshape(n, heads, c)
    if mean:
        _, _, d_v = gga_local_attn_bwd(fwd["desc"], None, None, None, None, None, d3, topo)
    else:
        d_q, d_k, d_v = gga_local_attn_bwd(fwd["desc"], fwd["q"], fwd["k"], fwd["v"], fwd["out3"], fwd["lse"], d3,
                                           topo)
    dv2 = d_v.view(n, n_rel * width)
    res = dict(d_w_v=gga_linear(x, dv2, trans_a=True), d_w_q=None, d_w_k=None)
    d_x = gga_linear(dv2, w_v, trans_b=True)
    if not mean:
        dq2, dk2 = d_q.view(n, width), d_k.view(n, n_rel * width)
        res["d_w_q"] = gga_linear(x, dq2, trans_a=True)
        res["d_w_k"] = gga_linear(x, dk2, trans_a=True)
        gga_linear_accumulate(dq2, w_q, d_x, trans_b=True)
        gga_linear_accumulate(dk2, w_k, d_x, trans_b=True)
    res["d_x"] = d_x
    return res


__all__ = ["gat_forward", "gat_backward", "gated_layer_forward", "gated_layer_backward", "relation_topology",
           "relation_forward", "relation_backward", "GGA_BF16"]
