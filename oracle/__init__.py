"""Plain CPU oracle for neighbor-restricted multi-head graph attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does, and
the two share no code.  Graph loops live in ``oracle.c`` (plain C, fp64, OpenMP
over rows); the dense steps (projections, the global linear branch, the gate,
LayerNorm) are written here with numpy in float64, a matmul being the only
library primitive used as a step.

Conventions.  An edge e: u -> v has source u (keys, values) and target v
(query, softmax group).  Node tensors are [N, H, C]; heads are contiguous
chunks of the feature axis and are normalised independently.

Parity status of each function (what pins it) is listed in its docstring.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIB names another build of oracle.c to load (the sanitizer test uses it)
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "_oracle.so")
_lib = None

SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined"]

SLOPE = 0.2  # LeakyReLU negative slope of the GAT score
LN_EPS = 1e-5
GLOBAL_EPS = 1e-6


def build(force: bool = True, path: str | None = None, sanitize: bool = False) -> str:
    """Compile oracle.c with gcc into _oracle.so (or `path`); with sanitize=True the host
    code is built with AddressSanitizer and UndefinedBehaviorSanitizer."""
    path = path or _LIB_PATH
    if force or not os.path.exists(path):
        tmp = path + ".tmp"
        opt = SANITIZE_FLAGS if sanitize else ["-O2"]
        subprocess.check_call(["gcc", *opt, "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, path)
    return path


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        stale = not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
        if stale and "ORACLE_LIB" not in os.environ:
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.orc_coo_to_csr.argtypes = [i32, i64, P, P, P, P, P]
        L.orc_coo_to_csr.restype = ctypes.c_int
        L.orc_local_fwd.argtypes = [ctypes.c_int, i32, i32, i32, P, P, P, P, P, f64, f64, P, P, P, i64, P, P]
        L.orc_local_fwd.restype = None
        L.orc_local_bwd.argtypes = [ctypes.c_int, i32, i32, i32, P, P, P, P, P, P, P, P, f64, f64, P, P, P, P,
                                    P, P, P, i64, P, P, i64, P, P]
        L.orc_local_bwd.restype = None
        L.orc_edge_values.argtypes = [i32, P, P, i64, P]
        L.orc_edge_values.restype = None
        L.orc_edge_values_bwd.argtypes = [i32, i32, P, P, P, P]
        L.orc_edge_values_bwd.restype = None
        L.orc_batch_edges.argtypes = [i32, P, P, P, P, P, P]
        L.orc_batch_edges.restype = i64
        L.orc_relation_fwd.argtypes = [ctypes.c_int, i32, i32, i32, P, P, P, P, P, P, P, f64, P, i64, P, P]
        L.orc_relation_fwd.restype = None
        L.orc_relation_bwd.argtypes = [ctypes.c_int, i32, i32, i32, i32, P, P, P, P, P, P, P, P, f64, P, P, P]
        L.orc_relation_bwd.restype = None
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_set_threads.restype = None
        L.orc_threads.argtypes = []
        L.orc_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def threads() -> int:
    return int(lib().orc_threads())


def set_threads(n: int) -> None:
    """Thread count of the C loops (OpenMP); results do not depend on it."""
    lib().orc_set_threads(int(n))


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


# --------------------------------------------------------------------------- CSR


def coo_to_csr(n: int, key, other):
    """Stable counting sort by key: (row_ptr[n+1], col[E] = other[eid], eid[E]).

    Tinymesh "Sparse attention experiment", section "Target softmax" (reductions
    traverse the destination CSR; COO order is kept).  Pinned by a library stable
    argsort and the histogram closed form."""
    key, other = _i32(key), _i32(other)
    e = key.shape[0]
    row_ptr = np.zeros(n + 1, np.int32)
    col = np.zeros(e, np.int32)
    eid = np.zeros(e, np.int32)
    rc = lib().orc_coo_to_csr(n, e, _p(key), _p(other), _p(row_ptr), _p(col), _p(eid))
    if rc != 0:
        raise ValueError("edge endpoint out of range")
    return row_ptr, col, eid


def batch_edges(node_ptr, edge_ptr, src_local, dst_local):
    """Packs a batch of B graphs into one block-diagonal graph over the packed node axis
    (Gated Local-Global Graph Attention, Implementation notes note 1: batched X with one
    sparse adjacency list per graph).  Graph b owns nodes node_ptr[b] .. node_ptr[b+1]-1
    and COO entries edge_ptr[b] .. edge_ptr[b+1]-1, whose endpoints are local ids in
    [0, n_b); they become local id + node_ptr[b].  An endpoint outside [0, n_b) is written
    as -1 and counted.  Returns (src, dst, bad).  Pinned by the block-diagonal assembly of
    per-graph adjacency matrices (library)."""
    node_ptr, edge_ptr = _i32(node_ptr), _i32(edge_ptr)
    src_local, dst_local = _i32(src_local), _i32(dst_local)
    e = src_local.shape[0]
    src = np.empty(e, np.int32)
    dst = np.empty(e, np.int32)
    bad = lib().orc_batch_edges(node_ptr.shape[0] - 1, _p(node_ptr), _p(edge_ptr), _p(src_local), _p(dst_local),
                                _p(src), _p(dst))
    return src, dst, int(bad)


class Graph:
    """Fixed topology: the COO list and both CSRs the oracle derives from it."""

    def __init__(self, n: int, src, dst):
        self.n = int(n)
        self.src, self.dst = _i32(src), _i32(dst)
        self.row_ptr, self.col, self.eid = coo_to_csr(self.n, self.dst, self.src)
        self.row_ptr_s, self.col_s, self.eid_s = coo_to_csr(self.n, self.src, self.dst)

    @property
    def e(self) -> int:
        return int(self.src.shape[0])


# --------------------------------------------------------------------------- local attention


def _rows(rows):
    if rows is None:
        return None, None
    r = _i32(rows)
    return r, r.shape[0]


def local_fwd_dot(q, k, v, g: Graph, scale: float, rows=None):
    """Dot-product local branch ("Gated Local-Global Graph Attention", Key formulas, L_i):
    per destination and head, softmax over in-edges of scale * q_v.k_u, weights applied
    to v_u.  Returns out [R,H,C] and lse [R,H] (R = len(rows) or N).

    Pinned by: masked scaled_dot_product_attention on dense graphs (library), the
    complete-graph reduction to dense multi-head attention, and invariants."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, hh, c = q.shape
    r, nr = _rows(rows)
    nr = n if r is None else nr
    out = np.empty((nr, hh, c), np.float64)
    lse = np.empty((nr, hh), np.float64)
    lib().orc_local_fwd(0, n, hh, c, _p(q), _p(k), _p(v), _p(g.row_ptr), _p(g.col), scale, 0.0, None, None, _p(r),
                        nr, _p(out), _p(lse))
    return out, lse


def local_fwd_add(s_src, s_dst, hf, g: Graph, slope: float = SLOPE, rows=None, s_edge=None):
    """GAT additive local attention (Tinymesh "Sparse attention experiment", sections
    "Composition" and "Multiple heads are composition"): score LeakyReLU(s_src[u] + s_dst[v]),
    target softmax, weighted sum of hf[u].  With s_edge [E,H] (COO order) the logit gains
    the edge's own term (learned edge features, as in the GATConv the page's reference
    contract follows).  Pinned by the two exact witnesses; the edge term by the masked dense
    formulation and by its equivalence to a per-source shift when sources are unique."""
    s_src, s_dst, hf = _f64(s_src), _f64(s_dst), _f64(hf)
    n, hh, c = hf.shape
    r, nr = _rows(rows)
    nr = n if r is None else nr
    out = np.empty((nr, hh, c), np.float64)
    lse = np.empty((nr, hh), np.float64)
    se = None if s_edge is None else _f64(s_edge).reshape(-1, hh)
    lib().orc_local_fwd(1, n, hh, c, _p(s_dst), _p(s_src), _p(hf), _p(g.row_ptr), _p(g.col), 0.0, slope, _p(se),
                        _p(g.eid), _p(r), nr, _p(out), _p(lse))
    return out, lse


def _local_bwd(mode, qs, ks, val, d_out, g: Graph, scale, slope, rows_d, rows_s, s_edge=None):
    qs, ks, val, d_out = _f64(qs), _f64(ks), _f64(val), _f64(d_out)
    n, hh, c = val.shape
    se = None if s_edge is None else _f64(s_edge).reshape(-1, hh)
    d_edge = None if s_edge is None else np.zeros((g.e, hh), np.float64)
    w = c if mode == 0 else 1
    rd, nd = _rows(rows_d)
    rs, ns = _rows(rows_s)
    nd = n if rd is None else nd
    ns = n if rs is None else ns
    lse = np.empty((n, hh), np.float64)
    dd = np.empty((n, hh), np.float64)
    d_qs = np.empty((nd, hh, w), np.float64)
    d_ks = np.empty((ns, hh, w), np.float64)
    d_val = np.empty((ns, hh, c), np.float64)
    lib().orc_local_bwd(mode, n, hh, c, _p(qs), _p(ks), _p(val), _p(d_out), _p(g.row_ptr), _p(g.col),
                        _p(g.row_ptr_s), _p(g.col_s), scale, slope, _p(se), _p(g.eid), _p(g.eid_s), _p(d_edge),
                        _p(lse), _p(dd), _p(rd), nd, _p(d_qs), _p(rs), ns, _p(d_ks), _p(d_val))
    if mode == 1:
        d_qs, d_ks = d_qs[..., 0], d_ks[..., 0]
    return dict(lse=lse, D=dd, d_q=d_qs, d_k=d_ks, d_v=d_val, d_edge=d_edge)


def local_bwd_dot(q, k, v, d_out, g: Graph, scale: float, rows_d=None, rows_s=None):
    """First-order gradients of sum(out * d_out) for the dot-product branch: dq over the
    destination CSR, dk and dv over the CSR by source.  Softmax gradient with the detached
    maximum (Tinymesh "Target softmax").  Pinned by autograd through masked dense attention
    (library) and central finite differences of local_fwd_dot."""
    return _local_bwd(0, q, k, v, d_out, g, scale, 0.0, rows_d, rows_s)


def local_bwd_add(s_src, s_dst, hf, d_out, g: Graph, slope: float = SLOPE, rows_d=None, rows_s=None, s_edge=None):
    """Gradients for the additive branch: d s_dst (destination CSR), d s_src and the
    aggregation part of d hf (CSR by source); with an edge term also d s_edge [E,H] (COO
    order; dz_e itself).  Pinned by the exact witnesses and by autograd through the dense
    formulation."""
    r = _local_bwd(1, s_dst, s_src, hf, d_out, g, 0.0, slope, rows_d, rows_s, s_edge)
    return dict(lse=r["lse"], D=r["D"], d_s_dst=r["d_q"], d_s_src=r["d_k"], d_hf=r["d_v"], d_s_edge=r["d_edge"])


# --------------------------------------------------------------------------- endpoint projection


def edge_values(x, endpoint):
    """out[e] = x[endpoint[e]] (Tinymesh "Endpoint projection").  Pinned by numpy indexing."""
    x = _f64(x)
    n = x.shape[0]
    w = int(np.prod(x.shape[1:])) if x.ndim > 1 else 1
    ep = _i32(endpoint)
    out = np.empty((ep.shape[0], w), np.float64)
    lib().orc_edge_values(w, _p(x.reshape(n, w)), _p(ep), ep.shape[0], _p(out))
    return out.reshape((ep.shape[0],) + x.shape[1:])


def edge_values_bwd(d_edge, endpoint, n: int):
    """dx[u] = sum of d_edge[e] over edges with endpoint[e] == u, via the CSR keyed by the
    endpoint (Tinymesh "Endpoint projection").  Pinned by numpy's unbuffered add.at."""
    d_edge = _f64(d_edge)
    e = d_edge.shape[0]
    w = int(np.prod(d_edge.shape[1:])) if d_edge.ndim > 1 else 1
    row_ptr, _, eid = coo_to_csr(n, endpoint, np.zeros(e, np.int32))
    dx = np.empty((n, w), np.float64)
    lib().orc_edge_values_bwd(n, w, _p(row_ptr), _p(eid), _p(d_edge.reshape(e, w)), _p(dx))
    return dx.reshape((n,) + d_edge.shape[1:])


# --------------------------------------------------------------------------- GAT layer


def gat_coefficients(x, w, a_s, a_t):
    """H = X W viewed as [N,K,C]; s_src[n,k] = a_s[k].H[n,k]; s_dst with a_t (Tinymesh
    "Composition": one source and one target coefficient per node and head)."""
    x, w, a_s, a_t = _f64(x), _f64(w), _f64(a_s), _f64(a_t)
    hh, c = a_s.shape
    hf = (x @ w).reshape(x.shape[0], hh, c)
    s_src = (hf * a_s[None]).sum(-1)
    s_dst = (hf * a_t[None]).sum(-1)
    return hf, s_src, s_dst


def edge_coefficients(f, w_e, a_e):
    """Learned edge features of the score (GATConv with edge features, the reference contract
    the Tinymesh page adopts; the page lists them as not yet covered): HE = F W_e viewed as
    [E,K,C] (no bias) and s_edge[e,k] = a_e[k].HE[e,k], added to the edge's logit."""
    f, w_e, a_e = _f64(f), _f64(w_e), _f64(a_e)
    hh, c = a_e.shape
    he = (f @ w_e).reshape(f.shape[0], hh, c)
    return he, (he * a_e[None]).sum(-1)


def gat_forward(x, w, a_s, a_t, g: Graph, slope: float = SLOPE, concat: bool = True, edge=None):
    """Multi-head GAT layer output plus intermediates: heads concatenated [N, K*C], or with
    concat=False averaged over heads [N, C] (head averaging, listed by the Tinymesh page
    as not yet covered).  edge = dict(f [E,Fe] in COO order, w_e [Fe,K*C], a_e [K,C]) adds
    the learned edge term to every logit."""
    hf, s_src, s_dst = gat_coefficients(x, w, a_s, a_t)
    he = s_edge = None
    if edge is not None:
        he, s_edge = edge_coefficients(edge["f"], edge["w_e"], edge["a_e"])
    out, lse = local_fwd_add(s_src, s_dst, hf, g, slope, s_edge=s_edge)
    res = out.reshape(out.shape[0], -1) if concat else out.mean(1)
    return dict(out=res, out3=out, hf=hf, s_src=s_src, s_dst=s_dst, lse=lse, he=he, s_edge=s_edge)


def gat_backward(x, w, a_s, a_t, d_out, g: Graph, slope: float = SLOPE, concat: bool = True, edge=None):
    """dX, dW, da_s, da_t (and with edge features dF, dW_e, da_e) of sum(out * d_out).
    Chain: with head averaging each head receives d_out / K; the local backward gives
    d s_src, d s_dst, d s_edge and the aggregation part of dH; the coefficient maps add
    a_s d s_src + a_t d s_dst (and a_e d s_edge for HE); then dW = X^T dH, dX = dH W^T,
    dW_e = F^T dHE, dF = dHE W_e^T."""
    x, w, a_s, a_t = _f64(x), _f64(w), _f64(a_s), _f64(a_t)
    hf, s_src, s_dst = gat_coefficients(x, w, a_s, a_t)
    n, hh, c = hf.shape
    if concat:
        d3 = _f64(d_out).reshape(n, hh, c)
    else:
        d3 = np.repeat(_f64(d_out)[:, None, :] / hh, hh, axis=1)
    he = s_edge = None
    if edge is not None:
        he, s_edge = edge_coefficients(edge["f"], edge["w_e"], edge["a_e"])
    r = local_bwd_add(s_src, s_dst, hf, d3, g, slope, s_edge=s_edge)
    d_hf = r["d_hf"] + a_s[None] * r["d_s_src"][..., None] + a_t[None] * r["d_s_dst"][..., None]
    da_s = (r["d_s_src"][..., None] * hf).sum(0)
    da_t = (r["d_s_dst"][..., None] * hf).sum(0)
    dh = d_hf.reshape(n, hh * c)
    res = dict(d_x=dh @ w.T, d_w=x.T @ dh, d_a_s=da_s, d_a_t=da_t, d_hf=d_hf, d_s_src=r["d_s_src"],
               d_s_dst=r["d_s_dst"])
    if edge is not None:
        f, w_e, a_e = _f64(edge["f"]), _f64(edge["w_e"]), _f64(edge["a_e"])
        d_se = r["d_s_edge"]
        d_he = (d_se[..., None] * a_e[None]).reshape(f.shape[0], hh * c)
        res.update(d_s_edge=d_se, d_a_e=(d_se[..., None] * he).sum(0), d_w_e=f.T @ d_he, d_f=d_he @ w_e.T)
    return res


# --------------------------------------------------------------------------- relation-typed edges

REL_SOFTMAX = 0  # softmax weighting of scaled q_v . k_{u,r} (GiGL "edge_type_attention")
REL_MEAN = 1  # every in-edge weighs 1/deg(v) (GiGL "edge_type_linear")


def relation_of_segments(e: int, segments, n_rel: int):
    """Relation of each packed edge row from host-side (relation, start, end) segments
    (GiGL pull request "Support relation message modes on the packed
    GraphTransformerEncoder path", section "Approach": relation edges travel as packed
    rows with per-relation segments).  Segments are taken in order; each starts where the
    previous one ended (the first at 0, the last ends at e), may be empty, and names a
    relation in [0, n_rel).  Anything else raises ValueError.  Pinned by a brute-force
    membership loop."""
    rel = np.empty(int(e), np.int32)
    pos = 0
    for r, start, end in segments:
        r, start, end = int(r), int(start), int(end)
        if start != pos or end < start or end > e or not 0 <= r < n_rel:
            raise ValueError(f"bad relation segment ({r}, {start}, {end})")
        rel[start:end] = r
        pos = end
    if pos != e:
        raise ValueError("relation segments do not cover the edge list")
    return rel


def relation_rows(src, rel, n: int, n_rel: int):
    """Row of the stacked per-relation projection that edge e reads: a projection of all
    nodes by the R relation transforms side by side is [N, R*W], which viewed as
    [N*R, W] holds x_u W^r in row u*R + r.  A source outside [0, n) gives -1 and is
    counted.  This is a layout convention, not a formula of the pages; pinned by indexing
    the stacked projection (library matmul) against the per-relation products."""
    src, rel = _i32(src), _i32(rel)
    ok = (src >= 0) & (src < n)
    out = np.where(ok, src.astype(np.int64) * n_rel + rel, -1).astype(np.int32)
    return out, int((~ok).sum())


def relation_projections(x, w_q, w_k, w_v, heads: int):
    """q = X W_Q [N,H,C] (None when w_q is None) and the per-relation key and message
    transforms key[r] = X W_K^r, val[r] = X W_V^r, each [R,N,H,C] (GiGL "Approach":
    per-relation transforms).  w_k, w_v are [R, d, H*C]; w_k may be None."""
    x = _f64(x)
    n = x.shape[0]
    w_v = _f64(w_v)
    n_rel, _, width = w_v.shape
    c = width // heads
    val = np.stack([x @ w_v[r] for r in range(n_rel)]).reshape(n_rel, n, heads, c)
    q = None if w_q is None else (x @ _f64(w_q)).reshape(n, heads, c)
    key = None if w_k is None else np.stack([x @ _f64(w_k)[r] for r in range(n_rel)]).reshape(n_rel, n, heads, c)
    return q, key, val


def relation_attention(q, key, val, src, dst, rel, mode: int, scale=None, rows=None):
    """Relation-typed message aggregation (GiGL "Approach": per-relation transforms, mean
    or softmax weighting, scatter-add).  Edge e: u -> v of relation r carries val[r, u];
    in softmax mode its head-h score is scale * q[v,h] . key[r,u,h] and the weights of
    v's in-edges (all relations together) are their softmax; in mean mode each weighs
    1/deg(v).  Returns out [R',H,C] and lse [R',H] for rows (all N by default); a row
    with no in-edges gets 0 and -inf.  Pinned by autograd through a dense masked
    formulation (library), the one-relation reduction to plain dot attention, a
    scatter-mean (library) and relabelling invariance."""
    val = _f64(val)
    n_rel, n, hh, c = val.shape
    if scale is None:
        scale = c ** -0.5
    row_ptr, col, eid = coo_to_csr(n, dst, src)
    rel = _i32(rel)
    r, nr = _rows(rows)
    nr = n if r is None else nr
    out = np.empty((nr, hh, c), np.float64)
    lse = np.empty((nr, hh), np.float64)
    qd = None if mode == REL_MEAN else _f64(q)
    kd = None if mode == REL_MEAN else _f64(key)
    lib().orc_relation_fwd(mode, n, hh, c, _p(qd), _p(kd), _p(val), _p(row_ptr), _p(col), _p(rel), _p(eid),
                           float(scale), _p(r), nr, _p(out), _p(lse))
    return out, lse


def relation_attention_bwd(q, key, val, d_out, src, dst, rel, mode: int, scale=None):
    """Gradients of sum(out * d_out) for relation_attention: d_q [N,H,C] and d_key,
    d_val [R,N,H,C] (d_q, d_key are None in mean mode, whose weights are constants)."""
    val = _f64(val)
    n_rel, n, hh, c = val.shape
    if scale is None:
        scale = c ** -0.5
    row_ptr, col, eid = coo_to_csr(n, dst, src)
    rel = _i32(rel)
    d_val = np.empty_like(val)
    d_q = d_key = qd = kd = None
    if mode == REL_SOFTMAX:
        qd, kd = _f64(q), _f64(key)
        d_q, d_key = np.empty_like(qd), np.empty_like(kd)
    lib().orc_relation_bwd(mode, n, n_rel, hh, c, _p(qd), _p(kd), _p(val), _p(_f64(d_out)), _p(row_ptr), _p(col),
                           _p(rel), _p(eid), float(scale), _p(d_q), _p(d_key), _p(d_val))
    return dict(d_q=d_q, d_key=d_key, d_val=d_val)


def relation_forward(x, w_q, w_k, w_v, src, dst, rel, heads: int, mode: int, rows=None):
    """Relation message layer: the projections then relation_attention.  Returns out
    [N, H*C] (rows only, when given) with the intermediates."""
    q, key, val = relation_projections(x, w_q if mode == REL_SOFTMAX else None,
                                       w_k if mode == REL_SOFTMAX else None, w_v, heads)
    out, lse = relation_attention(q, key, val, src, dst, rel, mode, rows=rows)
    return dict(out=out.reshape(out.shape[0], -1), lse=lse, q=q, key=key, val=val)


def relation_backward(x, w_q, w_k, w_v, src, dst, rel, heads: int, mode: int, d_out):
    """dX, dW_Q, dW_K, dW_V of sum(out * d_out): the attention gradients, then for each
    transform dW = X^T dY and dX = sum of dY W^T (dW_Q, dW_K are None in mean mode)."""
    x = _f64(x)
    n = x.shape[0]
    soft = mode == REL_SOFTMAX
    q, key, val = relation_projections(x, w_q if soft else None, w_k if soft else None, w_v, heads)
    n_rel, _, hh, c = val.shape
    g = relation_attention_bwd(q, key, val, _f64(d_out).reshape(n, hh, c), src, dst, rel, mode)
    w_v = _f64(w_v)
    dv = g["d_val"].reshape(n_rel, n, hh * c)
    d_w_v = np.stack([x.T @ dv[r] for r in range(n_rel)])
    d_x = sum(dv[r] @ w_v[r].T for r in range(n_rel))
    res = dict(d_w_v=d_w_v, d_w_q=None, d_w_k=None, d_q=g["d_q"], d_key=g["d_key"], d_val=g["d_val"])
    if soft:
        w_q, w_k = _f64(w_q), _f64(w_k)
        dq = g["d_q"].reshape(n, hh * c)
        dk = g["d_key"].reshape(n_rel, n, hh * c)
        res["d_w_q"] = x.T @ dq
        res["d_w_k"] = np.stack([x.T @ dk[r] for r in range(n_rel)])
        d_x = d_x + dq @ w_q.T + sum(dk[r] @ w_k[r].T for r in range(n_rel))
    res["d_x"] = d_x
    return res


# --------------------------------------------------------------------------- gated local-global layer


def phi(x):
    """phi = elu + 1 ("Gated Local-Global Graph Attention", Implementation notes)."""
    x = _f64(x)
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def global_linear(q, k, v, eps: float = GLOBAL_EPS):
    """Global branch per head ("Gated Local-Global Graph Attention", Key formulas, G_i):
    S = sum_j phi(k_j) v_j^T [H,r,r], z = sum_j phi(k_j) [H,r],
    G_i = phi(q_i)^T S / (phi(q_i)^T z + eps) [N,H,r].
    Pinned by the dense O(N^2) kernelised form."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    pq, pk = phi(q), phi(k)
    # per-head products as batched matrix products over the head axis ([H, ., .] operands)
    s = pk.transpose(1, 2, 0) @ v.transpose(1, 0, 2)  # S[h] = phi(K_h)^T V_h
    z = pk.sum(0)
    num = (pq.transpose(1, 0, 2) @ s).transpose(1, 0, 2)  # num[i, h] = phi(q_ih)^T S[h]
    den = (pq * z[None]).sum(-1) + eps
    return s, z, num / den[..., None]


def global_linear_seg(q, k, v, node_ptr, eps: float = GLOBAL_EPS):
    """The global branch over a batch of graphs packed along the node axis: graph b owns
    rows node_ptr[b] .. node_ptr[b+1]-1 and its statistics S_b, z_b sum over its own nodes
    only, so G_i = phi(q_i)^T S_b / (phi(q_i)^T z_b + eps) for i in graph b (Key formulas,
    per graph of the batch).  A graph with no node has S_b = 0, z_b = 0.
    Returns S [B,H,r,r], z [B,H,r], G [N,H,r].  Pinned by the dense kernelised form with a
    same-graph mask."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, hh, r = q.shape
    ptr = np.asarray(node_ptr, np.int64)
    b = ptr.shape[0] - 1
    s = np.zeros((b, hh, r, r))
    z = np.zeros((b, hh, r))
    glob = np.zeros((n, hh, r))
    for i in range(b):
        lo, hi = int(ptr[i]), int(ptr[i + 1])
        if hi > lo:
            s[i], z[i], glob[lo:hi] = global_linear(q[lo:hi], k[lo:hi], v[lo:hi], eps)
    return s, z, glob


def gate(x, w_g, b_g):
    """g_i = sigmoid(x_i . w_g + b_g), one scalar per node (Key formulas)."""
    t = _f64(x) @ _f64(w_g) + float(b_g)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-t))


def combine(gv, loc, glob):
    """Y_i = g_i L_i + (1 - g_i) G_i (Key formulas)."""
    gv = _f64(gv)[:, None]
    return gv * _f64(loc) + (1.0 - gv) * _f64(glob)


def layer_norm(a, gamma, beta, eps: float = LN_EPS):
    """Textbook LayerNorm over the last axis with biased variance."""
    a = _f64(a)
    mu = a.mean(-1, keepdims=True)
    var = ((a - mu) ** 2).mean(-1, keepdims=True)
    return _f64(gamma) * (a - mu) / np.sqrt(var + eps) + _f64(beta)


def gated_layer(p: dict, g: Graph, heads: int, eps: float = GLOBAL_EPS, rows=None, node_ptr=None):
    """The full layer of "Gated Local-Global Graph Attention" (Implementation notes, item 2):
    Q,K,V = X W_{Q,K,V}; local masked softmax per head; phi = elu+1 global branch;
    g = sigmoid(X w_g + b_g); out = LayerNorm(X + W_o(g L + (1-g) G)).
    ``rows`` restricts the per-node outputs (the global statistics S, z always use all
    nodes).  ``node_ptr`` [B+1] makes the input a batch of B graphs packed along the node
    axis (Implementation notes, note 1: a batched X with one adjacency list per graph): the
    graph g must then be the block-diagonal union (batch_edges) and S, z are per graph
    (global_linear_seg), shape [B, H, r, r] and [B, H, r].  Returns a dict of every
    intermediate, in float64."""
    x = _f64(p["x"])
    n, d = x.shape
    r = d // heads
    q = (x @ _f64(p["w_q"])).reshape(n, heads, r)
    k = (x @ _f64(p["w_k"])).reshape(n, heads, r)
    v = (x @ _f64(p["w_v"])).reshape(n, heads, r)
    loc, lse = local_fwd_dot(q, k, v, g, 1.0 / np.sqrt(r), rows=rows)
    xr = x if rows is None else x[np.asarray(rows)]
    if node_ptr is None:
        pk = phi(k)
        s = pk.transpose(1, 2, 0) @ v.transpose(1, 0, 2)  # S[h] = phi(K_h)^T V_h
        z = pk.sum(0)
        qr = q if rows is None else q[np.asarray(rows)]
        pq = phi(qr)
        num = (pq.transpose(1, 0, 2) @ s).transpose(1, 0, 2)  # phi(q_i)^T S[h]
        glob = num / ((pq * z[None]).sum(-1) + eps)[..., None]
    else:
        s, z, glob = global_linear_seg(q, k, v, node_ptr, eps)
        if rows is not None:
            glob = glob[np.asarray(rows)]
    gv = gate(xr, p["w_g"], p["b_g"])
    y = combine(gv, loc.reshape(-1, d), glob.reshape(-1, d))
    pre = xr + y @ _f64(p["w_o"])
    out = layer_norm(pre, p["gamma"], p["beta"])
    return dict(q=q, k=k, v=v, local=loc.reshape(-1, d), lse=lse, S=s, z=z, glob=glob.reshape(-1, d), gate=gv, y=y,
                pre=pre, out=out)


# --------------------------------------------------------------------------- gated layer backward


def phi_grad(x):
    """d phi / dx for phi = elu + 1: 1 for x > 0, exp(x) otherwise."""
    x = _f64(x)
    return np.where(x > 0.0, 1.0, np.exp(np.minimum(x, 0.0)))


def layer_norm_bwd(a, gamma, d_out, eps: float = LN_EPS):
    """Backward of out = gamma (a - mu)/sqrt(var + eps) + beta over the last axis:
    returns d a, d gamma, d beta (textbook LayerNorm derivative)."""
    a, gamma, d_out = _f64(a), _f64(gamma), _f64(d_out)
    mu = a.mean(-1, keepdims=True)
    inv = 1.0 / np.sqrt(((a - mu) ** 2).mean(-1, keepdims=True) + eps)
    xh = (a - mu) * inv
    dxh = d_out * gamma
    da = inv * (dxh - dxh.mean(-1, keepdims=True) - xh * (dxh * xh).mean(-1, keepdims=True))
    return da, (d_out * xh).sum(0), d_out.sum(0)


def global_linear_bwd(q, k, v, d_g, eps: float = GLOBAL_EPS):
    """Backward of the global branch G_i = phi(q_i)^T S / (phi(q_i)^T z + eps), S = sum_j
    phi(k_j) v_j^T, z = sum_j phi(k_j) ("Gated Local-Global Graph Attention", Key
    formulas), per head, by the chain rule: with num_i = phi(q_i)^T S and den_i the
    denominator, d num_i = dG_i / den_i and d den_i = -(dG_i . G_i) / den_i; then
    d phi(q_i) = S d num_i + z d den_i, dS = sum_i phi(q_i) d num_i^T, dz = sum_i phi(q_i) d den_i,
    d phi(k_j) = dS v_j + dz, dv_j = dS^T phi(k_j), and dq = d phi(q) phi'(q), dk likewise."""
    q, k, v, d_g = _f64(q), _f64(k), _f64(v), _f64(d_g)
    pq, pk = phi(q), phi(k)
    # per-head products as batched matrix products over the head axis; t() moves the node
    # axis behind the head axis ([N, H, r] -> [H, N, r]) and back
    t = lambda a: a.transpose(1, 0, 2)  # noqa: E731
    s = pk.transpose(1, 2, 0) @ t(v)  # S[h] = phi(K_h)^T V_h
    z = pk.sum(0)
    num = t(t(pq) @ s)
    den = (pq * z[None]).sum(-1) + eps
    gg = num / den[..., None]
    dnum = d_g / den[..., None]
    dden = -(d_g * gg).sum(-1) / den
    dpq = t(t(dnum) @ s.transpose(0, 2, 1)) + z[None] * dden[..., None]  # S dnum_i
    ds = pq.transpose(1, 2, 0) @ t(dnum)  # sum_i phi(q_i) dnum_i^T
    dz = (pq * dden[..., None]).sum(0)
    dpk = t(t(v) @ ds.transpose(0, 2, 1)) + dz[None]  # dS v_j + dz
    dv = t(t(pk) @ ds)  # dS^T phi(k_j)
    return dict(d_q=dpq * phi_grad(q), d_k=dpk * phi_grad(k), d_v=dv, d_S=ds, d_z=dz)


def global_linear_seg_bwd(q, k, v, d_g, node_ptr, eps: float = GLOBAL_EPS):
    """Backward of global_linear_seg: global_linear_bwd on each graph of the batch
    (graphs share no statistics, so their gradients are independent).  Returns d_q, d_k,
    d_v [N,H,r] and d_S [B,H,r,r], d_z [B,H,r].  Pinned by autograd through the masked dense
    kernelised form."""
    q, k, v, d_g = _f64(q), _f64(k), _f64(v), _f64(d_g)
    n, hh, r = q.shape
    ptr = np.asarray(node_ptr, np.int64)
    b = ptr.shape[0] - 1
    out = dict(d_q=np.zeros((n, hh, r)), d_k=np.zeros((n, hh, r)), d_v=np.zeros((n, hh, r)),
               d_S=np.zeros((b, hh, r, r)), d_z=np.zeros((b, hh, r)))
    for i in range(b):
        lo, hi = int(ptr[i]), int(ptr[i + 1])
        if hi > lo:
            res = global_linear_bwd(q[lo:hi], k[lo:hi], v[lo:hi], d_g[lo:hi], eps)
            for key in ("d_q", "d_k", "d_v"):
                out[key][lo:hi] = res[key]
            out["d_S"][i], out["d_z"][i] = res["d_S"], res["d_z"]
    return out


def gated_layer_backward(p: dict, g: Graph, heads: int, d_out, eps: float = GLOBAL_EPS, ln_eps: float = LN_EPS,
                         node_ptr=None):
    """First-order gradients of sum(out * d_out) for the gated local-global layer (the
    forward of gated_layer): dX and the gradients of W_Q, W_K, W_V, W_o, w_g, b_g, gamma,
    beta.  Chain: LayerNorm -> residual and W_o -> gate and combination -> local branch
    (local_bwd_dot) and global branch (global_linear_bwd, per graph with node_ptr) ->
    projections."""
    f = gated_layer(p, g, heads, eps, node_ptr=node_ptr)
    x = _f64(p["x"])
    n, d = x.shape
    r = d // heads
    d_pre, d_gamma, d_beta = layer_norm_bwd(f["pre"], p["gamma"], d_out, ln_eps)
    dy = d_pre @ _f64(p["w_o"]).T
    d_wo = f["y"].T @ d_pre
    gv = f["gate"][:, None]
    d_loc = gv * dy
    d_glob = (1.0 - gv) * dy
    d_gate = (dy * (f["local"] - f["glob"])).sum(-1)
    d_t = d_gate * f["gate"] * (1.0 - f["gate"])
    d_wg = x.T @ d_t
    d_bg = d_t.sum()
    loc = local_bwd_dot(f["q"], f["k"], f["v"], d_loc.reshape(n, heads, r), g, 1.0 / np.sqrt(r))
    if node_ptr is None:
        glb = global_linear_bwd(f["q"], f["k"], f["v"], d_glob.reshape(n, heads, r), eps)
    else:
        glb = global_linear_seg_bwd(f["q"], f["k"], f["v"], d_glob.reshape(n, heads, r), node_ptr, eps)
    dq = (loc["d_q"] + glb["d_q"]).reshape(n, d)
    dk = (loc["d_k"] + glb["d_k"]).reshape(n, d)
    dv = (loc["d_v"] + glb["d_v"]).reshape(n, d)
    d_x = d_pre + np.outer(d_t, _f64(p["w_g"])) + dq @ _f64(p["w_q"]).T + dk @ _f64(p["w_k"]).T + \
        dv @ _f64(p["w_v"]).T
    return dict(d_x=d_x, d_w_q=x.T @ dq, d_w_k=x.T @ dk, d_w_v=x.T @ dv, d_w_o=d_wo, d_w_g=d_wg, d_b_g=d_bg,
                d_gamma=d_gamma, d_beta=d_beta, d_pre=d_pre, d_y=dy, d_local=d_loc, d_glob=d_glob, d_gate=d_gate,
                d_t=d_t, d_q=dq, d_k=dk, d_v=dv, fwd=f)
