"""The C-ABI library loads and exports every entry point include/gga.h declares, and
its host-side argument checks reject bad calls before anything reaches a GPU.

No call here passes its checks, so nothing is launched and no GPU is needed."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "sparse_graph_attention_amd", "libgga.so")


def _header_symbols():
    txt = open(os.path.join(ROOT, "include", "gga.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gga_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import importlib.util

        spec = importlib.util.spec_from_file_location("gga_build", os.path.join(ROOT, "sparse_graph_attention_amd",
                                                                                "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return ctypes.CDLL(LIB)


def test_header_declares_the_boundary():
    syms = _header_symbols()
    for name in ["gga_coo_to_csr", "gga_edge_values", "gga_local_attn_fwd", "gga_local_attn_bwd",
                 "gga_global_linear_fwd", "gga_gated_combine"]:
        assert name in syms


def test_every_declared_symbol_is_exported(lib):
    missing = [s for s in _header_symbols() if not hasattr(lib, s)]
    assert not missing, missing


def test_binding_names_match_header():
    import sparse_graph_attention_amd as g

    for s in _header_symbols():
        if s.endswith("_workspace") or s in ("gga_plan_bytes", "gga_plan_workspace"):
            assert hasattr(g.lib, s)
        else:
            assert callable(getattr(g, s)), s


def test_binding_refuses_to_import_without_the_library(tmp_path):
    """The binding has no fallback: a copy of the package without libgga.so fails to import."""
    import shutil
    import subprocess
    import sys

    pkg = tmp_path / "sparse_graph_attention_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "sparse_graph_attention_amd", "__init__.py"), pkg / "__init__.py")
    r = subprocess.run([sys.executable, "-c", "import sparse_graph_attention_amd"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libgga.so is missing" in r.stderr


def test_version_and_status(lib):
    lib.gga_abi_version.restype = ctypes.c_int
    lib.gga_status_string.restype = ctypes.c_char_p
    assert lib.gga_abi_version() == 4
    assert lib.gga_status_string(0) == b"ok"
    assert lib.gga_status_string(4).startswith(b"workspace")


def _desc(**kw):
    import sparse_graph_attention_amd as g

    d = dict(n=10, e=20, heads=2, head_dim=8, score=0, dtype=0)
    d.update(kw)
    return g.make_desc(d["n"], d["e"], d["heads"], d["head_dim"], d["score"], d["dtype"])


@pytest.mark.parametrize("bad,status", [
    (dict(n=-1), 1), (dict(heads=0), 1), (dict(head_dim=0), 1), (dict(e=-5), 1),
    (dict(e=1 << 31), 2), (dict(e=(1 << 31) - 4000), 2), (dict(score=7), 3), (dict(dtype=9), 3), (dict(heads=1, head_dim=1000), 3),
])
def test_fwd_rejects_bad_desc(bad, status):
    import sparse_graph_attention_amd as g

    d = _desc(**bad)
    fake = ctypes.c_void_p(256)
    rc = g.lib.gga_local_attn_fwd(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, None, None, 0, None)
    assert rc == status


@pytest.mark.parametrize("heads,c,dtype,ok", [
    (1, 512, 1, True), (1, 1024, 1, False),   # bf16: at most 64 lanes of 8 per head
    (1, 256, 0, True), (1, 512, 0, False),    # fp32: 64 lanes of 4
    (16, 64, 1, True), (24, 64, 1, False),    # at most two 64-lane slots
    (8, 64, 0, True), (12, 64, 0, False),
    (64, 1, 0, True), (65, 1, 0, False),      # scalar elements: one slot
    (1, 64, 0, True), (1, 65, 0, False),      # scalar path: 65 lanes for one head
])
def test_shape_limits(heads, c, dtype, ok):
    """The lane layouts cover heads x head_dim up to the limits the header states; one
    step past each is rejected as unsupported before any launch."""
    import sparse_graph_attention_amd as g

    d = _desc(heads=heads, head_dim=c, dtype=dtype)
    assert (g.lib.gga_local_attn_fwd_workspace(ctypes.byref(d)) > 0) == ok
    assert (g.lib.gga_local_attn_bwd_workspace(ctypes.byref(d)) > 0) == ok
    if not ok:
        fake = ctypes.c_void_p(256)
        assert g.lib.gga_local_attn_fwd(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, None, None, 0,
                                        None) == 3


def test_desc_rejects_negative_source_rows():
    import sparse_graph_attention_amd as g

    d = _desc()
    d.n_src = -3
    fake = ctypes.c_void_p(256)
    assert g.lib.gga_local_attn_fwd(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, None, None, 0,
                                    None) == 1
    assert g.lib.gga_local_attn_bwd_workspace(ctypes.byref(d)) == 0


def test_mean_mode_needs_no_query_or_key():
    """Mean weighting reads neither q nor k: NULL passes the pointer checks (the call then
    stops at the workspace check, before any launch)."""
    import sparse_graph_attention_amd as g

    d = _desc(e=5000, score=g.GGA_SCORE_MEAN)
    a = ctypes.c_void_p(4096)
    need = g.lib.gga_local_attn_fwd_workspace(ctypes.byref(d))
    assert need > 0
    assert g.lib.gga_local_attn_fwd(ctypes.byref(d), None, None, a, a, a, a, a, None, a, need - 1, None) == 4
    dd = _desc(e=5000, score=g.GGA_SCORE_DOT)
    assert g.lib.gga_local_attn_fwd(ctypes.byref(dd), None, None, a, a, a, a, a, None, a, 1 << 40, None) == 1
    nb = g.lib.gga_local_attn_bwd_workspace(ctypes.byref(d))
    assert nb > 0
    assert g.lib.gga_local_attn_bwd(ctypes.byref(d), None, None, None, None, None, a, a, a, a, a, a, a, None, None,
                                    a, a, nb - 1, None) == 4
    assert g.lib.gga_local_attn_bwd(ctypes.byref(d), None, None, None, None, None, a, a, a, a, a, a, a, None, None,
                                    None, a, nb, None) == 1


@pytest.mark.parametrize("segs,n,rels,e,status", [
    ([(0, 0, 5), (1, 5, 9)], 4, 2, 10, 1),    # does not reach e
    ([(0, 0, 5), (1, 6, 10)], 4, 2, 10, 1),   # gap
    ([(0, 0, 6), (1, 5, 10)], 4, 2, 10, 1),   # overlap
    ([(2, 0, 10)], 4, 2, 10, 1),              # relation out of range
    ([(-1, 0, 10)], 4, 2, 10, 1),
    ([(0, 0, 11)], 4, 2, 10, 1),              # beyond e
    ([(0, 0, 10)], 4, 0, 10, 1),              # no relations
    ([(0, 0, 10)], 1 << 29, 8, 10, 2),        # n * R beyond int32
])
def test_relation_sources_rejects(segs, n, rels, e, status):
    import sparse_graph_attention_amd as g

    a = ctypes.c_void_p(4096)
    flat = (ctypes.c_int32 * (3 * len(segs)))(*[x for t in segs for x in t])
    assert g.lib.gga_relation_sources(n, rels, e, a, a, len(segs), flat, a, a, None) == status


def test_fwd_rejects_null_and_misaligned_and_small_workspace():
    import sparse_graph_attention_amd as g

    d = _desc(e=5000)
    a = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4100)
    L = g.lib
    assert L.gga_local_attn_fwd(ctypes.byref(d), a, a, None, a, a, a, a, None, None, 0, None) == 1
    assert L.gga_local_attn_fwd(ctypes.byref(d), a, a, mis, a, a, a, a, None, None, 0, None) == 1
    need = L.gga_local_attn_fwd_workspace(ctypes.byref(d))
    assert need > 0
    assert L.gga_local_attn_fwd(ctypes.byref(d), a, a, a, a, a, a, a, None, a, need - 1, None) == 4


def test_csr_and_plan_checks():
    import sparse_graph_attention_amd as g

    L = g.lib
    a = ctypes.c_void_p(4096)
    assert L.gga_coo_to_csr(-1, 0, None, None, a, None, None, None, 0, None) == 1
    assert L.gga_coo_to_csr(4, 1 << 31, a, a, a, a, a, a, 1 << 40, None) == 2
    assert L.gga_coo_to_csr(4, 10, None, a, a, a, a, a, 1 << 40, None) == 1
    need = L.gga_coo_to_csr_workspace(100, 1000)
    assert need > 0
    assert L.gga_coo_to_csr(100, 1000, a, a, a, a, a, a, need - 1, None) == 4
    pb = L.gga_plan_bytes(100, 1000)
    assert L.gga_plan_build(100, 1000, a, a, pb - 1, a, 1 << 30, None) == 4
    assert L.gga_plan_status(None, 100, 1000, a, None) == 1
    assert L.gga_plan_status(a, 100, 1000, None, None) == 1
    assert L.gga_plan_status(a, -1, 1000, a, None) == 1
    assert L.gga_plan_status(a, 100, 1 << 31, a, None) == 2
    assert L.gga_validate_coo(3, 4, None, a, a, None) == 1


def test_workspaces_are_linear_not_quadratic():
    """No dense N x N or N x E carrier (Tinymesh "Endpoint projection": work and storage O(EH))."""
    import sparse_graph_attention_amd as g

    L = g.lib
    for n, e in [(1 << 20, 17 << 20), (1 << 21, 67 << 20)]:
        assert L.gga_coo_to_csr_workspace(n, e) < 64 * (n + e)
        assert L.gga_plan_bytes(n, e) < 64 * (n + e)
        d = _desc(n=n, e=e, heads=8, head_dim=64, dtype=1)
        assert L.gga_local_attn_fwd_workspace(ctypes.byref(d)) < 8 * e * 8 * 64


def test_noalloc_forward_refuses_inputs_beyond_its_scratch():
    """The allocation-free forward checks its fixed scratch size on the host, before any
    device work: a graph whose split-row partials would need more is refused."""
    import sparse_graph_attention_amd as g

    a = ctypes.c_void_p(4096)
    d = _desc(n=1000, e=1 << 30, heads=8, head_dim=64, dtype=1)
    assert g.lib.gga_local_attn_fwd_workspace(ctypes.byref(d)) > 96 << 20
    assert g.lib.gga_local_attn_fwd_noalloc(ctypes.byref(d), a, a, a, a, a, a, a, a, None) == g.GGA_ESCRATCH
    assert g.lib.gga_status_string(g.GGA_ESCRATCH) != g.lib.gga_status_string(99)


def test_fused_projection_checks():
    import sparse_graph_attention_amd as g

    L = g.lib
    a = ctypes.c_void_p(4096)
    assert L.gga_qkv_gate_proj(-1, 256, a, a, a, a, a, ctypes.c_float(0.0), a, a, a, a, None, 0, None) == 1
    assert L.gga_qkv_gate_proj(10, 256, a, a, None, a, a, ctypes.c_float(0.0), a, a, a, a, None, 0, None) == 1
    assert L.gga_qkv_gate_proj(0, 256, None, None, None, None, None, ctypes.c_float(0.0), None, None, None, None,
                               None, 0, None) == 0
    need = L.gga_qkv_proj_bwd_x_workspace(1000, 256)
    assert need >= 3 * 256 * 256 * 4
    assert L.gga_qkv_proj_bwd_x(1000, 256, a, a, a, a, a, a, None, None, a, a, need - 1, None) == 4
    assert L.gga_qkv_proj_bwd_x(1000, 0, a, a, a, a, a, a, None, None, a, a, need, None) == 1
    # the gate logit's share needs both its vectors
    assert L.gga_qkv_proj_bwd_x(1000, 256, a, a, a, a, a, a, a, None, a, a, need, None) == 1
    assert L.gga_qkv_proj_bwd_x(1000, 256, a, a, a, a, a, a, None, a, a, a, need, None) == 1
    # the combine backward: d_x_in and d_x_out together, or neither and d_logit
    cneed = L.gga_gated_combine_bwd_workspace(1000, 256)
    f0 = ctypes.c_float(0.0)
    assert L.gga_gated_combine_bwd(1000, 256, a, a, f0, 256, a, a, a, a, a, a, None, a, a, a, a, cneed, None) == 1
    assert L.gga_gated_combine_bwd(1000, 256, a, a, f0, 256, a, a, a, a, a, None, None, None, a, a, a, cneed,
                                   None) == 1
    assert L.gga_gated_combine_bwd(1000, 256, a, a, f0, 256, a, a, a, a, a, None, None, a, a, a, a, cneed - 1,
                                   None) == 4
    assert L.gga_gated_combine(10, 4, None, a, a, None, a, None) == 1


def test_global_branch_backward_checks():
    """The global branch's backward (with or without the forward's G) refuses bad shapes,
    missing tensors and a short workspace before launching anything; n = 0 is a no-op."""
    import sparse_graph_attention_amd as g

    L = g.lib
    a = ctypes.c_void_p(4096)
    eps = ctypes.c_float(1e-6)
    need = L.gga_global_linear_bwd_workspace(1000, 4, 64)
    assert need > 0
    for gfw in (None, a):
        assert L.gga_global_linear_bwd(-1, 4, 64, a, a, a, eps, a, a, a, gfw, a, a, a, a, need, None) == g.GGA_EINVAL
        assert L.gga_global_linear_bwd(1000, 4, 65, a, a, a, eps, a, a, a, gfw, a, a, a, a, need, None) == \
            g.GGA_EUNSUPPORTED
        assert L.gga_global_linear_bwd(1000, 4, 64, a, a, a, eps, a, a, None, gfw, a, a, a, a, need, None) == \
            g.GGA_EINVAL
        assert L.gga_global_linear_bwd(1000, 4, 64, a, a, a, eps, a, a, a, gfw, a, a, a, a, need - 1, None) == \
            g.GGA_EWORKSPACE
        assert L.gga_global_linear_bwd(0, 4, 64, None, None, None, eps, None, None, None, gfw, None, None, None,
                                       None, 0, None) == g.GGA_OK
        bneed = L.gga_global_linear_batch_workspace(1000, 3, 4, 64)
        assert L.gga_global_linear_batch_bwd(1000, 3, None, 4, 64, a, a, a, eps, a, a, a, gfw, a, a, a, a, bneed,
                                             None) == g.GGA_EINVAL
        assert L.gga_global_linear_batch_bwd(1000, 3, a, 4, 64, a, a, a, eps, a, a, a, gfw, a, a, a, a, bneed - 1,
                                             None) == g.GGA_EWORKSPACE
