"""Python binding of libgga: neighbor-restricted multi-head graph attention on MI355X.

Every function here has the name of the C entry point it wraps (include/gga.h) and
only marshals arguments: torch tensors become device pointers, the current HIP
stream is passed along, output and workspace tensors are allocated with torch when
the caller does not supply them, and a nonzero status raises GGAError.  All
arithmetic runs in the HIP kernels of libgga.so; importing this package fails if
the library has not been built (``python sparse_graph_attention_amd/build.py``).
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgga.so")

GGA_OK, GGA_EINVAL, GGA_ERANGE, GGA_EUNSUPPORTED, GGA_EWORKSPACE, GGA_EHIP, GGA_ESCRATCH = range(7)
GGA_F32, GGA_BF16 = 0, 1
GGA_SCORE_DOT, GGA_SCORE_ADDITIVE, GGA_SCORE_MEAN = 0, 1, 2


class GGAError(RuntimeError):
    def __init__(self, name: str, status: int):
        self.status = status
        super().__init__(f"{name} failed: {gga_status_string(status)} ({status})")


class gga_local_desc(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("e", ctypes.c_int64),
        ("head_dim", ctypes.c_int32),
        ("score", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("negative_slope", ctypes.c_float),
        ("n_src", ctypes.c_int32),
    ]


ABI_VERSION = 4


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python sparse_graph_attention_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    D = ctypes.POINTER(gga_local_desc)
    sig = {
        "gga_abi_version": ([], ctypes.c_int),
        "gga_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "gga_validate_coo": ([i32, i64, P, P, P, P], ctypes.c_int),
        "gga_coo_to_csr_workspace": ([i32, i64], sz),
        "gga_coo_to_csr": ([i32, i64, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "gga_plan_bytes": ([i32, i64], sz),
        "gga_plan_workspace": ([i32, i64], sz),
        "gga_plan_build": ([i32, i64, P, P, sz, P, sz, P], ctypes.c_int),
        "gga_plan_status": ([P, i32, i64, P, P], ctypes.c_int),
        "gga_local_attn_fwd_workspace": ([D], sz),
        "gga_local_attn_fwd": ([D, P, P, P, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "gga_local_attn_fwd_noalloc": ([D, P, P, P, P, P, P, P, P, P], ctypes.c_int),
        "gga_local_attn_bwd_workspace": ([D], sz),
        "gga_local_attn_bwd": ([D, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "gga_edge_values": ([i32, i32, i32, P, i64, P, P, P], ctypes.c_int),
        "gga_edge_values_bwd": ([i32, i32, i64, P, P, P, P, P], ctypes.c_int),
        "gga_gat_coef_fwd": ([i32, i32, i32, P, P, P, P, P, P], ctypes.c_int),
        "gga_gat_coef_bwd_workspace": ([i32, i32, i32], sz),
        "gga_gat_coef_bwd": ([i32, i32, i32, P, P, P, P, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "gga_linear_workspace": ([i32, i32, i32], sz),
        "gga_linear": ([i32, i32, i32, i32, i32, P, P, P, P, P, sz, P], ctypes.c_int),
        "gga_global_linear_workspace": ([i32, i32, i32], sz),
        "gga_global_linear_fwd": ([i32, i32, i32, P, P, P, f32, P, P, P, P, sz, P], ctypes.c_int),
        "gga_gated_combine": ([i32, i32, P, P, P, P, P, P], ctypes.c_int),
        "gga_qkv_gate_proj_workspace": ([i32, i32], sz),
        "gga_qkv_gate_proj": ([i32, i32, P, P, P, P, P, f32, P, P, P, P, P, sz, P], ctypes.c_int),
        "gga_qkv_proj_bwd_x_workspace": ([i32, i32], sz),
        "gga_qkv_proj_bwd_x": ([i32, i32, P, P, P, P, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "gga_add_layernorm": ([i32, i32, P, P, P, P, f32, P, P], ctypes.c_int),
        "gga_linear_accumulate": ([i32, i32, i32, i32, i32, P, P, P, P, sz, P], ctypes.c_int),
        "gga_add_layernorm_bwd_workspace": ([i32, i32], sz),
        "gga_add_layernorm_bwd": ([i32, i32, P, P, P, f32, P, P, P, P, P, sz, P], ctypes.c_int),
        "gga_gated_combine_bwd_workspace": ([i32, i32], sz),
        "gga_gated_combine_bwd": ([i32, i32, P, P, f32, i32, P, P, P, P, P, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "gga_global_linear_bwd_workspace": ([i32, i32, i32], sz),
        "gga_global_linear_bwd": ([i32, i32, i32, P, P, P, f32, P, P, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "gga_batch_edges": ([i32, P, P, i64, P, P, P, P, P, P], ctypes.c_int),
        "gga_relation_sources": ([i32, i32, i64, P, P, i32, P, P, P, P], ctypes.c_int),
        "gga_local_attn_fwd_edge_workspace": ([D], sz),
        "gga_local_attn_fwd_edge": ([D, P, P, P, P, P, P, P, P, P, P, P, sz, P], ctypes.c_int),
        "gga_local_attn_bwd_edge_workspace": ([D], sz),
        "gga_local_attn_bwd_edge": ([D] + [P] * 20 + [sz, P], ctypes.c_int),
        "gga_head_mean": ([i32, i32, i32, P, P, P], ctypes.c_int),
        "gga_head_mean_bwd": ([i32, i32, i32, P, P, P], ctypes.c_int),
        "gga_global_linear_batch_workspace": ([i32, i32, i32, i32], sz),
        "gga_global_linear_batch_fwd": ([i32, i32, P, i32, i32, P, P, P, f32, P, P, P, P, sz, P], ctypes.c_int),
        "gga_global_linear_batch_bwd": ([i32, i32, P, i32, i32, P, P, P, f32, P, P, P, P, P, P, P, P, sz, P],
                                        ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    # the signatures above are those of this ABI version; a library built from other sources
    # would take the arguments differently
    if L.gga_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {L.gga_abi_version()}, this binding expects {ABI_VERSION}: "
                          "rebuild it with `python sparse_graph_attention_amd/build.py`")
    return L


lib = _load()


# --------------------------------------------------------------------------- marshalling helpers


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(name: str, rc: int) -> None:
    if rc != GGA_OK:
        raise GGAError(name, rc)


def _workspace(nbytes: int, device, ws=None):
    if nbytes == 0:
        return None
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise GGAError("workspace", GGA_EWORKSPACE)
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _row_width(t: torch.Tensor) -> int:
    """Elements per row of a node tensor [N, ...]."""
    w = 1
    for s in t.shape[1:]:
        w *= int(s)
    return w


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GGA_F32
    if t.dtype == torch.bfloat16:
        return GGA_BF16
    raise GGAError(f"dtype {t.dtype}", GGA_EUNSUPPORTED)


def gga_abi_version() -> int:
    return int(lib.gga_abi_version())


def gga_status_string(status: int) -> str:
    return lib.gga_status_string(int(status)).decode()


# --------------------------------------------------------------------------- graph


def gga_validate_coo(n: int, src: torch.Tensor, dst: torch.Tensor, d_bad=None, stream=None) -> torch.Tensor:
    d_bad = torch.empty(1, dtype=torch.int32, device=src.device) if d_bad is None else d_bad
    _check("gga_validate_coo", lib.gga_validate_coo(n, src.numel(), _ptr(src), _ptr(dst), _ptr(d_bad),
                                                    _stream(stream)))
    return d_bad


def gga_coo_to_csr(n: int, key: torch.Tensor, other: torch.Tensor, row_ptr=None, col=None, eid=None, ws=None,
                   stream=None):
    e = key.numel()
    dev = key.device
    row_ptr = torch.empty(n + 1, dtype=torch.int32, device=dev) if row_ptr is None else row_ptr
    col = torch.empty(e, dtype=torch.int32, device=dev) if col is None else col
    eid = torch.empty(e, dtype=torch.int32, device=dev) if eid is None else eid
    nb = lib.gga_coo_to_csr_workspace(n, e)
    ws = _workspace(nb, dev, ws)
    _check("gga_coo_to_csr", lib.gga_coo_to_csr(n, e, _ptr(key), _ptr(other), _ptr(row_ptr), _ptr(col), _ptr(eid),
                                                _ptr(ws), nb, _stream(stream)))
    return row_ptr, col, eid


def gga_plan_build(n: int, e: int, row_ptr: torch.Tensor, plan=None, ws=None, stream=None) -> torch.Tensor:
    dev = row_ptr.device
    pb = lib.gga_plan_bytes(n, e)
    plan = torch.empty(pb, dtype=torch.uint8, device=dev) if plan is None else plan
    wb = lib.gga_plan_workspace(n, e)
    ws = _workspace(wb, dev, ws)
    _check("gga_plan_build", lib.gga_plan_build(n, e, _ptr(row_ptr), _ptr(plan), plan.numel(), _ptr(ws), wb,
                                                _stream(stream)))
    return plan


def gga_plan_status(plan: torch.Tensor, n: int, e: int, stream=None) -> torch.Tensor:
    """Device int32 [1]: the plan's status for (n, e) (GGA_OK, GGA_ERANGE or GGA_EINVAL)."""
    st = torch.empty(1, dtype=torch.int32, device=plan.device)
    _check("gga_plan_status", lib.gga_plan_status(_ptr(plan), n, e, _ptr(st), _stream(stream)))
    return st


class Topology:
    """A fixed graph on the device: the CSR by destination with its plan and, when
    ``backward`` is set, the CSR by source with its plan (built by the entry points
    above; this class only keeps the tensors together).  Sources index n_src rows
    (default n), e.g. the (node, relation) rows of gga_relation_sources."""

    def __init__(self, n: int, src: torch.Tensor, dst: torch.Tensor, backward: bool = False, stream=None,
                 n_src: int | None = None):
        self.n = int(n)
        self.n_src = self.n if n_src is None else int(n_src)
        self.e = int(src.numel())
        self.src, self.dst = src, dst
        self.row_ptr, self.col, self.eid = gga_coo_to_csr(n, dst, src, stream=stream)
        self.plan = gga_plan_build(n, self.e, self.row_ptr, stream=stream)
        self.row_ptr_s = self.col_s = self.eid_s = self.plan_s = None
        if backward:
            self.build_source_csr(stream)

    def build_source_csr(self, stream=None):
        self.row_ptr_s, self.col_s, self.eid_s = gga_coo_to_csr(self.n_src, self.src, self.dst, stream=stream)
        self.plan_s = gga_plan_build(self.n_src, self.e, self.row_ptr_s, stream=stream)


# --------------------------------------------------------------------------- local attention


def make_desc(n, e, heads, head_dim, score, dtype, scale=None, negative_slope=0.2, n_src=0) -> gga_local_desc:
    if scale is None:
        scale = head_dim ** -0.5 if head_dim > 0 else 1.0
    return gga_local_desc(n, heads, e, head_dim, score, dtype, scale, negative_slope, n_src)


def gga_local_attn_fwd(desc: gga_local_desc, qs, ks, v, row_ptr, col, plan, out=None, lse=None, want_lse=True,
                       ws=None, stream=None):
    dev = v.device
    if out is None:
        out = torch.empty(desc.n, desc.heads, desc.head_dim, dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(desc.n, desc.heads, dtype=torch.float32, device=dev)
    nb = lib.gga_local_attn_fwd_workspace(ctypes.byref(desc))
    ws = _workspace(nb, dev, ws)
    _check("gga_local_attn_fwd", lib.gga_local_attn_fwd(ctypes.byref(desc), _ptr(qs), _ptr(ks), _ptr(v),
                                                        _ptr(row_ptr), _ptr(col), _ptr(plan), _ptr(out), _ptr(lse),
                                                        _ptr(ws), nb, _stream(stream)))
    return out, lse


def gga_local_attn_fwd_noalloc(desc: gga_local_desc, qs, ks, v, row_ptr, col, plan, out, lse=None, stream=None):
    """The allocation-free forward: the caller passes out (and lse, or None); nothing is
    allocated here or in the library (split-row partials use the library's fixed array)."""
    _check("gga_local_attn_fwd_noalloc", lib.gga_local_attn_fwd_noalloc(
        ctypes.byref(desc), _ptr(qs), _ptr(ks), _ptr(v), _ptr(row_ptr), _ptr(col), _ptr(plan), _ptr(out), _ptr(lse),
        _stream(stream)))
    return out, lse


def gga_local_attn_bwd(desc: gga_local_desc, qs, ks, v, out, lse, d_out, topo: Topology, d_qs=None, d_ks=None,
                       d_v=None, ws=None, stream=None):
    dev = d_out.device
    ns = desc.n_src if desc.n_src > 0 else desc.n
    if desc.score != GGA_SCORE_MEAN:
        tail = (desc.heads, desc.head_dim) if desc.score == GGA_SCORE_DOT else (desc.heads,)
        d_qs = torch.empty((desc.n,) + tail, dtype=torch.float32, device=dev) if d_qs is None else d_qs
        d_ks = torch.empty((ns,) + tail, dtype=torch.float32, device=dev) if d_ks is None else d_ks
    d_v = torch.empty(ns, desc.heads, desc.head_dim, dtype=torch.float32, device=dev) if d_v is None else d_v
    nb = lib.gga_local_attn_bwd_workspace(ctypes.byref(desc))
    ws = _workspace(nb, dev, ws)
    _check("gga_local_attn_bwd", lib.gga_local_attn_bwd(
        ctypes.byref(desc), _ptr(qs), _ptr(ks), _ptr(v), _ptr(out), _ptr(lse), _ptr(d_out), _ptr(topo.row_ptr),
        _ptr(topo.col), _ptr(topo.plan), _ptr(topo.row_ptr_s), _ptr(topo.col_s), _ptr(topo.plan_s), _ptr(d_qs),
        _ptr(d_ks), _ptr(d_v), _ptr(ws), nb, _stream(stream)))
    return d_qs, d_ks, d_v


# --------------------------------------------------------------------------- endpoint projection, GAT


def gga_edge_values(x: torch.Tensor, endpoint: torch.Tensor, out=None, stream=None):
    n = x.shape[0]
    width = x.numel() // max(n, 1) if n else (x.shape[1] if x.dim() > 1 else 1)
    e = endpoint.numel()
    out = torch.empty((e,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device) if out is None else out
    _check("gga_edge_values", lib.gga_edge_values(n, width, _dtype_code(x), _ptr(x), e, _ptr(endpoint), _ptr(out),
                                                  _stream(stream)))
    return out


def gga_edge_values_bwd(n: int, d_edge: torch.Tensor, row_ptr, eid, dx=None, stream=None):
    e = d_edge.shape[0]
    width = d_edge.numel() // max(e, 1) if e else (d_edge.shape[1] if d_edge.dim() > 1 else 1)
    dx = torch.empty((n,) + tuple(d_edge.shape[1:]), dtype=torch.float32, device=d_edge.device) if dx is None else dx
    _check("gga_edge_values_bwd", lib.gga_edge_values_bwd(n, width, e, _ptr(row_ptr), _ptr(eid), _ptr(d_edge),
                                                          _ptr(dx), _stream(stream)))
    return dx


def gga_gat_coef_fwd(hf: torch.Tensor, a_s: torch.Tensor, a_t, s_src=None, s_dst=None, stream=None):
    """a_t None: one coefficient per row (s_dst None)."""
    n, heads, c = hf.shape
    s_src = torch.empty(n, heads, dtype=torch.float32, device=hf.device) if s_src is None else s_src
    if a_t is not None and s_dst is None:
        s_dst = torch.empty(n, heads, dtype=torch.float32, device=hf.device)
    _check("gga_gat_coef_fwd", lib.gga_gat_coef_fwd(n, heads, c, _ptr(hf), _ptr(a_s), _ptr(a_t), _ptr(s_src),
                                                    _ptr(s_dst), _stream(stream)))
    return s_src, s_dst


def gga_gat_coef_bwd(hf, a_s, a_t, d_hf_attn, d_s_src, d_s_dst, d_hf=None, d_a_s=None, d_a_t=None, ws=None,
                     stream=None):
    n, heads, c = hf.shape
    dev = hf.device
    d_hf = torch.empty_like(hf) if d_hf is None else d_hf
    d_a_s = torch.empty(heads, c, dtype=torch.float32, device=dev) if d_a_s is None else d_a_s
    if a_t is not None and d_a_t is None:
        d_a_t = torch.empty(heads, c, dtype=torch.float32, device=dev)
    nb = lib.gga_gat_coef_bwd_workspace(n, heads, c)
    ws = _workspace(nb, dev, ws)
    _check("gga_gat_coef_bwd", lib.gga_gat_coef_bwd(n, heads, c, _ptr(hf), _ptr(a_s), _ptr(a_t), _ptr(d_hf_attn),
                                                    _ptr(d_s_src), _ptr(d_s_dst), _ptr(d_hf), _ptr(d_a_s),
                                                    _ptr(d_a_t), _ptr(ws), nb, _stream(stream)))
    return d_hf, d_a_s, d_a_t


# --------------------------------------------------------------------------- dense steps


def gga_linear(a: torch.Tensor, b: torch.Tensor, bias=None, trans_a=False, trans_b=False, out=None, ws=None,
               stream=None):
    m = a.shape[1] if trans_a else a.shape[0]
    k = a.shape[0] if trans_a else a.shape[1]
    n = b.shape[0] if trans_b else b.shape[1]
    out = torch.empty(m, n, dtype=torch.float32, device=a.device) if out is None else out
    nb = lib.gga_linear_workspace(m, k, n)
    ws = _workspace(nb, a.device, ws)
    _check("gga_linear", lib.gga_linear(m, k, n, int(trans_a), int(trans_b), _ptr(a), _ptr(b), _ptr(bias), _ptr(out),
                                        _ptr(ws), nb, _stream(stream)))
    return out


def gga_global_linear_fwd(q, k, v, eps=1e-6, s_out=None, z_out=None, g_out=None, ws=None, stream=None):
    n, heads, r = q.shape
    dev = q.device
    s_out = torch.empty(heads, r, r, dtype=torch.float32, device=dev) if s_out is None else s_out
    z_out = torch.empty(heads, r, dtype=torch.float32, device=dev) if z_out is None else z_out
    g_out = torch.empty(n, heads, r, dtype=torch.float32, device=dev) if g_out is None else g_out
    nb = lib.gga_global_linear_workspace(n, heads, r)
    ws = _workspace(nb, dev, ws)
    _check("gga_global_linear_fwd", lib.gga_global_linear_fwd(n, heads, r, _ptr(q), _ptr(k), _ptr(v), eps,
                                                              _ptr(s_out), _ptr(z_out), _ptr(g_out), _ptr(ws), nb,
                                                              _stream(stream)))
    return s_out, z_out, g_out


def gga_qkv_gate_proj(x, w_q, w_k, w_v, w_g, b_g: float, heads: int, ws=None, stream=None):
    """Q, K, V ([n, heads, d/heads] each) and the gate logit [n] from one product."""
    n, d = x.shape
    dev = x.device
    q, k, v = (torch.empty(n, heads, d // heads, dtype=torch.float32, device=dev) for _ in range(3))
    logit = torch.empty(n, dtype=torch.float32, device=dev)
    nb = lib.gga_qkv_gate_proj_workspace(n, d)
    ws = _workspace(nb, dev, ws)
    _check("gga_qkv_gate_proj", lib.gga_qkv_gate_proj(n, d, _ptr(x), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_g),
                                                      float(b_g), _ptr(q), _ptr(k), _ptr(v), _ptr(logit), _ptr(ws),
                                                      nb, _stream(stream)))
    return q, k, v, logit


def gga_qkv_proj_bwd_x(d_q, d_k, d_v, w_q, w_k, w_v, d_x, ws=None, stream=None, d_logit=None, w_g=None):
    """d_x += d_q W_Q^T + d_k W_K^T + d_v W_V^T (+ d_logit w_g^T when both are given;
    d_q, d_k, d_v viewed [n, d])."""
    n, d = d_x.shape
    nb = lib.gga_qkv_proj_bwd_x_workspace(n, d)
    ws = _workspace(nb, d_x.device, ws)
    _check("gga_qkv_proj_bwd_x", lib.gga_qkv_proj_bwd_x(n, d, _ptr(d_q), _ptr(d_k), _ptr(d_v), _ptr(w_q), _ptr(w_k),
                                                        _ptr(w_v), _ptr(d_logit), _ptr(w_g), _ptr(d_x), _ptr(ws), nb,
                                                        _stream(stream)))
    return d_x


def gga_gated_combine(gate_logit, l, g, gate_out=None, y=None, stream=None):
    n = gate_logit.shape[0]
    width = _row_width(l)
    y = torch.empty(n, width, dtype=torch.float32, device=l.device) if y is None else y
    gate_out = torch.empty(n, dtype=torch.float32, device=l.device) if gate_out is None else gate_out
    _check("gga_gated_combine", lib.gga_gated_combine(n, width, _ptr(gate_logit), _ptr(l), _ptr(g), _ptr(gate_out),
                                                      _ptr(y), _stream(stream)))
    return gate_out, y


def gga_add_layernorm(x, y, gamma, beta, eps=1e-5, out=None, stream=None):
    n, d = x.shape
    out = torch.empty_like(x) if out is None else out
    _check("gga_add_layernorm", lib.gga_add_layernorm(n, d, _ptr(x), _ptr(y), _ptr(gamma), _ptr(beta), eps,
                                                      _ptr(out), _stream(stream)))
    return out


# --------------------------------------------------------------------------- layer backward


def gga_linear_accumulate(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor, trans_a=False, trans_b=False, ws=None,
                          stream=None):
    m = a.shape[1] if trans_a else a.shape[0]
    k = a.shape[0] if trans_a else a.shape[1]
    n = b.shape[0] if trans_b else b.shape[1]
    nb = lib.gga_linear_workspace(m, k, n)
    ws = _workspace(nb, a.device, ws)
    _check("gga_linear_accumulate", lib.gga_linear_accumulate(m, k, n, int(trans_a), int(trans_b), _ptr(a), _ptr(b),
                                                              _ptr(out), _ptr(ws), nb, _stream(stream)))
    return out


def gga_add_layernorm_bwd(x, y, gamma, d_out, eps=1e-5, d_pre=None, d_gamma=None, d_beta=None, ws=None, stream=None):
    n, d = x.shape
    dev = x.device
    d_pre = torch.empty_like(x) if d_pre is None else d_pre
    d_gamma = torch.empty(d, dtype=torch.float32, device=dev) if d_gamma is None else d_gamma
    d_beta = torch.empty(d, dtype=torch.float32, device=dev) if d_beta is None else d_beta
    nb = lib.gga_add_layernorm_bwd_workspace(n, d)
    ws = _workspace(nb, dev, ws)
    _check("gga_add_layernorm_bwd", lib.gga_add_layernorm_bwd(n, d, _ptr(x), _ptr(y), _ptr(gamma), eps, _ptr(d_out),
                                                              _ptr(d_pre), _ptr(d_gamma), _ptr(d_beta), _ptr(ws), nb,
                                                              _stream(stream)))
    return d_pre, d_gamma, d_beta


def gga_gated_combine_bwd(x, w_g, b_g: float, l, g, d_y, d_x_in, d_l=None, d_g=None, d_x_out=None, d_w_g=None,
                          d_b_g=None, ws=None, stream=None, d_logit=None, want_logit=False):
    """Returns (d_l, d_g, d_x_out, d_w_g, d_b_g, d_logit).  With d_x_in None no input gradient is
    formed (d_x_out is None) and the [n] logit gradients are returned for the caller to add
    d_logit w_g^T itself; want_logit also returns them beside d_x_out."""
    n, d = x.shape
    dev = x.device
    width = _row_width(l)
    d_l = torch.empty(n, width, dtype=torch.float32, device=dev) if d_l is None else d_l
    d_g = torch.empty(n, width, dtype=torch.float32, device=dev) if d_g is None else d_g
    if d_x_in is not None and d_x_out is None:
        d_x_out = torch.empty_like(x)
    if (d_x_in is None or want_logit) and d_logit is None:
        d_logit = torch.empty(n, dtype=torch.float32, device=dev)
    d_w_g = torch.empty(d, dtype=torch.float32, device=dev) if d_w_g is None else d_w_g
    d_b_g = torch.empty(1, dtype=torch.float32, device=dev) if d_b_g is None else d_b_g
    nb = lib.gga_gated_combine_bwd_workspace(n, d)
    ws = _workspace(nb, dev, ws)
    _check("gga_gated_combine_bwd", lib.gga_gated_combine_bwd(n, d, _ptr(x), _ptr(w_g), float(b_g), width, _ptr(l),
                                                              _ptr(g), _ptr(d_y), _ptr(d_l), _ptr(d_g), _ptr(d_x_in),
                                                              _ptr(d_x_out), _ptr(d_logit), _ptr(d_w_g), _ptr(d_b_g),
                                                              _ptr(ws), nb, _stream(stream)))
    return d_l, d_g, d_x_out, d_w_g, d_b_g, d_logit


def gga_global_linear_bwd(q, k, v, s, z, d_g, d_q, d_k, d_v, eps=1e-6, ws=None, stream=None, g_fw=None):
    """Adds the global branch's gradients into d_q, d_k, d_v (all [n, H, r] fp32).  g_fw:
    the forward's G ([n, H, r] fp32), or None to form it again from S."""
    n, heads, r = q.shape
    nb = lib.gga_global_linear_bwd_workspace(n, heads, r)
    ws = _workspace(nb, q.device, ws)
    _check("gga_global_linear_bwd", lib.gga_global_linear_bwd(n, heads, r, _ptr(q), _ptr(k), _ptr(v), eps, _ptr(s),
                                                              _ptr(z), _ptr(d_g), _ptr(g_fw), _ptr(d_q), _ptr(d_k),
                                                              _ptr(d_v), _ptr(ws), nb, _stream(stream)))
    return d_q, d_k, d_v


# --------------------------------------------------------------------------- batches of graphs


def gga_batch_edges(node_ptr: torch.Tensor, edge_ptr: torch.Tensor, src_local: torch.Tensor, dst_local: torch.Tensor,
                    src=None, dst=None, d_bad=None, stream=None):
    """Packs per-graph local COO lists into the block-diagonal list; returns (src, dst, d_bad)."""
    batch = node_ptr.numel() - 1
    e = src_local.numel()
    dev = src_local.device
    src = torch.empty(e, dtype=torch.int32, device=dev) if src is None else src
    dst = torch.empty(e, dtype=torch.int32, device=dev) if dst is None else dst
    d_bad = torch.empty(1, dtype=torch.int32, device=dev) if d_bad is None else d_bad
    _check("gga_batch_edges", lib.gga_batch_edges(batch, _ptr(node_ptr), _ptr(edge_ptr), e, _ptr(src_local),
                                                  _ptr(dst_local), _ptr(src), _ptr(dst), _ptr(d_bad),
                                                  _stream(stream)))
    return src, dst, d_bad


def gga_relation_sources(n: int, relations: int, src: torch.Tensor, dst: torch.Tensor, segments, src_rel=None,
                         d_bad=None, stream=None):
    """Source rows of relation-typed edges; ``segments`` is host data: (relation, start,
    end) triples.  Returns (src_rel, d_bad)."""
    e = src.numel()
    dev = src.device
    seg = (ctypes.c_int32 * max(1, 3 * len(segments)))(*[int(x) for t in segments for x in t])
    src_rel = torch.empty(e, dtype=torch.int32, device=dev) if src_rel is None else src_rel
    d_bad = torch.empty(1, dtype=torch.int32, device=dev) if d_bad is None else d_bad
    _check("gga_relation_sources", lib.gga_relation_sources(n, relations, e, _ptr(src), _ptr(dst), len(segments),
                                                            seg, _ptr(src_rel), _ptr(d_bad), _stream(stream)))
    return src_rel, d_bad


def gga_global_linear_batch_fwd(node_ptr, q, k, v, eps=1e-6, s_out=None, z_out=None, g_out=None, ws=None,
                                stream=None):
    n, heads, r = q.shape
    batch = node_ptr.numel() - 1
    dev = q.device
    s_out = torch.empty(batch, heads, r, r, dtype=torch.float32, device=dev) if s_out is None else s_out
    z_out = torch.empty(batch, heads, r, dtype=torch.float32, device=dev) if z_out is None else z_out
    g_out = torch.empty(n, heads, r, dtype=torch.float32, device=dev) if g_out is None else g_out
    nb = lib.gga_global_linear_batch_workspace(n, batch, heads, r)
    ws = _workspace(nb, dev, ws)
    _check("gga_global_linear_batch_fwd",
           lib.gga_global_linear_batch_fwd(n, batch, _ptr(node_ptr), heads, r, _ptr(q), _ptr(k), _ptr(v), eps,
                                           _ptr(s_out), _ptr(z_out), _ptr(g_out), _ptr(ws), nb, _stream(stream)))
    return s_out, z_out, g_out


def gga_global_linear_batch_bwd(node_ptr, q, k, v, s, z, d_g, d_q, d_k, d_v, eps=1e-6, ws=None, stream=None,
                                g_fw=None):
    """Adds the per-graph global branch's gradients into d_q, d_k, d_v (g_fw as in
    gga_global_linear_bwd)."""
    n, heads, r = q.shape
    batch = node_ptr.numel() - 1
    nb = lib.gga_global_linear_batch_workspace(n, batch, heads, r)
    ws = _workspace(nb, q.device, ws)
    _check("gga_global_linear_batch_bwd",
           lib.gga_global_linear_batch_bwd(n, batch, _ptr(node_ptr), heads, r, _ptr(q), _ptr(k), _ptr(v), eps,
                                           _ptr(s), _ptr(z), _ptr(d_g), _ptr(g_fw), _ptr(d_q), _ptr(d_k), _ptr(d_v),
                                           _ptr(ws), nb, _stream(stream)))
    return d_q, d_k, d_v


# --------------------------------------------------------------------------- GAT variants


def gga_local_attn_fwd_edge(desc: gga_local_desc, s_dst, s_src, hf, s_edge, topo: Topology, out=None, lse=None,
                            ws=None, stream=None):
    """Additive local attention whose logits include s_edge [E,H] (COO order)."""
    dev = hf.device
    out = torch.empty(desc.n, desc.heads, desc.head_dim, dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty(desc.n, desc.heads, dtype=torch.float32, device=dev) if lse is None else lse
    nb = lib.gga_local_attn_fwd_edge_workspace(ctypes.byref(desc))
    ws = _workspace(nb, dev, ws)
    _check("gga_local_attn_fwd_edge", lib.gga_local_attn_fwd_edge(
        ctypes.byref(desc), _ptr(s_dst), _ptr(s_src), _ptr(hf), _ptr(s_edge), _ptr(topo.row_ptr), _ptr(topo.col),
        _ptr(topo.eid), _ptr(topo.plan), _ptr(out), _ptr(lse), _ptr(ws), nb, _stream(stream)))
    return out, lse


def gga_local_attn_bwd_edge(desc: gga_local_desc, s_dst, s_src, hf, s_edge, out, lse, d_out, topo: Topology,
                            d_s_dst=None, d_s_src=None, d_hf=None, d_s_edge=None, ws=None, stream=None):
    """Returns d s_dst, d s_src, d hf (aggregation part) and d s_edge (COO order)."""
    dev = hf.device
    n, heads, c = desc.n, desc.heads, desc.head_dim
    ns = desc.n_src if desc.n_src > 0 else n
    d_s_dst = torch.empty(n, heads, dtype=torch.float32, device=dev) if d_s_dst is None else d_s_dst
    d_s_src = torch.empty(ns, heads, dtype=torch.float32, device=dev) if d_s_src is None else d_s_src
    d_hf = torch.empty(ns, heads, c, dtype=torch.float32, device=dev) if d_hf is None else d_hf
    d_s_edge = torch.empty(desc.e, heads, dtype=torch.float32, device=dev) if d_s_edge is None else d_s_edge
    nb = lib.gga_local_attn_bwd_edge_workspace(ctypes.byref(desc))
    ws = _workspace(nb, dev, ws)
    _check("gga_local_attn_bwd_edge", lib.gga_local_attn_bwd_edge(
        ctypes.byref(desc), _ptr(s_dst), _ptr(s_src), _ptr(hf), _ptr(s_edge), _ptr(out), _ptr(lse), _ptr(d_out),
        _ptr(topo.row_ptr), _ptr(topo.col), _ptr(topo.eid), _ptr(topo.plan), _ptr(topo.row_ptr_s), _ptr(topo.col_s),
        _ptr(topo.eid_s), _ptr(topo.plan_s), _ptr(d_s_dst), _ptr(d_s_src), _ptr(d_hf), _ptr(d_s_edge), _ptr(ws), nb,
        _stream(stream)))
    return d_s_dst, d_s_src, d_hf, d_s_edge


def gga_head_mean(x: torch.Tensor, out=None, stream=None):
    """x [n,H,C] -> mean over heads [n,C]."""
    n, heads, c = x.shape
    out = torch.empty(n, c, dtype=torch.float32, device=x.device) if out is None else out
    _check("gga_head_mean", lib.gga_head_mean(n, heads, c, _ptr(x), _ptr(out), _stream(stream)))
    return out


def gga_head_mean_bwd(d_out: torch.Tensor, heads: int, d_in=None, stream=None):
    n, c = d_out.shape
    d_in = torch.empty(n, heads, c, dtype=torch.float32, device=d_out.device) if d_in is None else d_in
    _check("gga_head_mean_bwd", lib.gga_head_mean_bwd(n, heads, c, _ptr(d_out), _ptr(d_in), _stream(stream)))
    return d_in
