"""The allocation-free forward (gga_local_attn_fwd_noalloc, for callers that cannot
allocate) against the forward that takes a caller workspace: bit-identical outputs on two
calls in a row, the second on a smaller graph of another shape, both graphs with rows split
into chunks (so the fixed scratch array holds partial states) and checked against the
oracle as well; an input needing more than the fixed array is refused before any launch."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, i32, node_pair

pytestmark = pytest.mark.gpu


def _case(g, n, seed, hubs, heads, c, dtype):
    src, dst = synth.mixed_degree_graph(n, seed, hubs=hubs)
    print(f"noalloc n={n} e={src.size} H={heads} C={c} {dtype}", flush=True)
    topo = g.Topology(n, i32(src), i32(dst))
    rng = np.random.default_rng(seed)
    qh, qd = node_pair(rng.standard_normal((n, heads, c)).astype(np.float32), dtype)
    kh, kd = node_pair(rng.standard_normal((n, heads, c)).astype(np.float32), dtype)
    vh, vd = node_pair(rng.standard_normal((n, heads, c)).astype(np.float32), dtype)
    desc = g.make_desc(n, src.size, heads, c, g.GGA_SCORE_DOT, g.GGA_BF16 if dtype == "bf16" else g.GGA_F32)
    assert g.lib.gga_local_attn_fwd_workspace(ctypes.byref(desc)) > 0  # split rows use scratch
    ref, ref_lse = g.gga_local_attn_fwd(desc, qd, kd, vd, topo.row_ptr, topo.col, topo.plan)
    out = torch.full((n, heads, c), 7.0, device="cuda")
    lse = torch.full((n, heads), 7.0, device="cuda")
    g.gga_local_attn_fwd_noalloc(desc, qd, kd, vd, topo.row_ptr, topo.col, topo.plan, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
    want, want_lse = oracle.local_fwd_dot(qh, kh, vh, oracle.Graph(n, src, dst), c ** -0.5)
    assert_close(out.cpu().numpy(), want, dtype, "out")
    assert_close(lse.cpu().numpy(), want_lse, dtype, "lse")


def test_noalloc_matches_workspace_forward(g=None):
    import sparse_graph_attention_amd as g

    _case(g, 6000, 31, (9000, 4097, 2050, 1025, 700, 65), 8, 32, "bf16")
    _case(g, 2000, 32, (3000, 1100), 2, 16, "f32")  # a smaller input, another shape


def test_noalloc_refuses_inputs_beyond_its_scratch():
    import sparse_graph_attention_amd as g

    desc = g.make_desc(1000, 1 << 30, 8, 64, g.GGA_SCORE_DOT, g.GGA_BF16)
    a = ctypes.c_void_p(4096)
    assert g.lib.gga_local_attn_fwd_noalloc(ctypes.byref(desc), a, a, a, a, a, a, a, a, None) == g.GGA_ESCRATCH
