"""GPU parity sweep of the local attention over every lane layout the kernels pick: elements
per lane (16-byte vectors or single elements), lanes per head 1..64, rows narrower than a
wavefront (2..64 edge groups) or one or two full slots, in fp32 and bf16, dot and additive
scores.  Each layout runs on two graphs: light rows of a few edges (each edge group of a
wavefront then takes a row of its own) and light rows of about 40 edges (the rows run one
after another, every group on each), both with isolated targets and hubs that take the
workgroup and the chunk-and-merge paths.  Forward (out, lse) and both backward passes are
compared with the oracle at the standard tolerances."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, i32, node_pair

pytestmark = pytest.mark.gpu

# (H, C): lanes per row 1, 2, 4, 8, 16, 32, 64 and two slots; 16-byte and single-element rows
LAYOUTS = [(1, 1), (1, 4), (2, 3), (1, 16), (4, 8), (8, 8), (3, 32), (8, 32), (5, 24), (12, 32), (16, 64),
           (1, 256), (2, 256), (64, 1)]


@pytest.fixture(scope="module")
def g():
    import sparse_graph_attention_amd as m

    return m


def _graphs():
    short = synth.mixed_degree_graph(400, 71, hubs=(1100, 70), background=2)
    long_ = synth.mixed_degree_graph(400, 72, hubs=(1100, 70), background=40)
    return {"short": short, "long": long_}


@pytest.mark.parametrize("score", [0, 1])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layout_sweep(g, dtype, score):
    n = 400
    checked = 0
    for gname, (src, dst) in _graphs().items():
        og = oracle.Graph(n, src, dst)
        topo = g.Topology(n, i32(src), i32(dst), backward=True)
        for heads, c in LAYOUTS:
            code = g.GGA_BF16 if dtype == "bf16" else g.GGA_F32
            scale = c ** -0.5
            desc = g.make_desc(n, src.size, heads, c, score, code, scale)
            if g.lib.gga_local_attn_fwd_workspace(desc) == 0:
                continue  # a shape the kernels do not take (checked on the CPU side)
            print(f"sweep {gname} H={heads} C={c} {dtype} {'dot' if score == 0 else 'add'}", flush=True)
            rng = np.random.default_rng(heads * 1000 + c)
            vh, vd = node_pair(rng.standard_normal((n, heads, c)).astype(np.float32), dtype)
            d_out = rng.standard_normal((n, heads, c)).astype(np.float32)
            if score == g.GGA_SCORE_DOT:
                qh, qd = node_pair(rng.standard_normal((n, heads, c)).astype(np.float32), dtype)
                kh, kd = node_pair(rng.standard_normal((n, heads, c)).astype(np.float32), dtype)
            else:
                qh = rng.standard_normal((n, heads)).astype(np.float32)
                kh = rng.standard_normal((n, heads)).astype(np.float32)
                qd, kd = torch.from_numpy(qh).cuda(), torch.from_numpy(kh).cuda()
            out, lse = g.gga_local_attn_fwd(desc, qd, kd, vd, topo.row_ptr, topo.col, topo.plan)
            dq, dk, dv = g.gga_local_attn_bwd(desc, qd, kd, vd, out, lse, torch.from_numpy(d_out).cuda(), topo)
            torch.cuda.synchronize()
            if score == g.GGA_SCORE_DOT:
                ro, rl = oracle.local_fwd_dot(qh, kh, vh, og, scale)
                r = oracle.local_bwd_dot(qh, kh, vh, d_out, og, scale)
                refs = (r["d_q"], r["d_k"], r["d_v"])
            else:
                ro, rl = oracle.local_fwd_add(kh, qh, vh, og, 0.2)
                r = oracle.local_bwd_add(kh, qh, vh, d_out, og, 0.2)
                refs = (r["d_s_dst"], r["d_s_src"], r["d_hf"])
            what = f"{gname} H={heads} C={c}"
            assert_close(out.cpu().numpy(), ro, dtype, "out " + what)
            assert_close(lse.cpu().numpy(), rl, dtype, "lse " + what)
            for got, want, nm in zip((dq, dk, dv), refs, ("d_q", "d_k", "d_v")):
                assert_close(got.cpu().numpy(), want, dtype, f"{nm} {what}")
            checked += 1
    taken = [hc for hc in LAYOUTS
             if g.lib.gga_local_attn_fwd_workspace(g.make_desc(n, 1, hc[0], hc[1], score, code, 1.0)) > 0]
    # every layout runs, but fp32 rows of 16 x 64 (past the two-slot limit of 512 elements)
    assert len(taken) == len(LAYOUTS) - (dtype == "f32") and checked == 2 * len(taken)
