"""GPU parity of the COO -> CSR build and the degree plan: bit-exact against the oracle.

Edge cases: empty graph, one node, isolated rows, duplicates, a row longer than one
radix tile, every workload graph at its full size (the CSR by destination and by source),
and index validation."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import i32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import sparse_graph_attention_amd as m

    return m


def _csr_exact(g, n, key, other):
    print(f"csr n={n} e={key.size}", flush=True)
    rp, col, eid = g.gga_coo_to_csr(n, i32(key), i32(other))
    torch.cuda.synchronize()
    ref = oracle.coo_to_csr(n, key, other)
    np.testing.assert_array_equal(rp.cpu().numpy(), ref[0])
    np.testing.assert_array_equal(eid.cpu().numpy(), ref[2])
    np.testing.assert_array_equal(col.cpu().numpy(), ref[1])


@pytest.mark.parametrize("n,m,seed,iso", [(1, 0, 0, 0), (1, 9, 1, 0), (2, 3, 2, 0), (257, 5000, 3, 10),
                                          (1000, 20000, 4, 50), (70000, 300000, 5, 1000)])
def test_csr_small(g, n, m, seed, iso):
    src, dst = synth.random_multigraph(n, m, seed, isolated=iso)
    _csr_exact(g, n, dst, src)
    _csr_exact(g, n, src, dst)


def test_csr_empty(g):
    rp, col, eid = g.gga_coo_to_csr(5, i32(np.zeros(0)), i32(np.zeros(0)))
    assert rp.cpu().tolist() == [0] * 6
    rp, _, _ = g.gga_coo_to_csr(0, i32(np.zeros(0)), i32(np.zeros(0)))
    assert rp.cpu().tolist() == [0]


def test_csr_hub_rows(g):
    src, dst = synth.mixed_degree_graph(5000, 1, hubs=(50000, 9000, 4097, 4096, 1025))
    _csr_exact(g, 5000, dst, src)


@pytest.mark.parametrize("ident", [1, 2, 3, 4, 5])
def test_csr_workloads(g, ident):
    n = synth.WORKLOADS[ident].n
    src, dst = synth.workload_graph(ident)
    _csr_exact(g, n, dst, src)
    if ident in (2, 5):
        _csr_exact(g, n, src, dst)


@pytest.mark.parametrize("case", ["one_target", "last_target", "sorted", "reversed", "sparse_keys"])
def test_csr_key_patterns(g, case):
    """Key layouts that stress the radix passes and the row_ptr written with the last pass:
    every edge on one row (each 64-item round of one digit), keys already sorted or
    reversed, and a few keys spread over many rows (most tile runs empty, long gaps of empty
    rows between runs and after the largest key)."""
    rng = np.random.default_rng(17)
    n, e = 300_000, 200_000
    other = rng.integers(0, n, e).astype(np.int32)
    if case == "one_target":
        key = np.zeros(e, np.int32)
    elif case == "last_target":
        key = np.full(e, n - 1, np.int32)
    elif case == "sorted":
        key = np.sort(rng.integers(0, n, e)).astype(np.int32)
    elif case == "reversed":
        key = np.sort(rng.integers(0, n, e))[::-1].astype(np.int32)
    else:
        key = rng.choice(np.array([3, 4096, 77_777, 150_001, 262_143], np.int32), e)
    _csr_exact(g, n, key, other)


@pytest.mark.parametrize("n", [127, 128, 129, 16_384, 16_385, (1 << 21) + 1])
def test_csr_pass_counts(g, n):
    """Node counts at the edges of the digit-pass counts (key bits 7, 8, 14, 15 and 22:
    one to four passes of at most 7 bits)."""
    src, dst = synth.random_multigraph(n, 150_000, 23, isolated=n // 10)
    _csr_exact(g, n, dst, src)


def test_validate_coo(g):
    src = np.array([0, 1, 5, -1, 2], np.int32)
    dst = np.array([1, 7, 2, 0, 2], np.int32)
    bad = g.gga_validate_coo(5, i32(src), i32(dst))
    assert int(bad.item()) == 3
    bad = g.gga_validate_coo(8, i32(src), i32(dst))
    assert int(bad.item()) == 1


def _plan_tables(plan, n, e):
    """The header, light list, chunk table and heavy list of a plan buffer (layout of
    plan.hpp: 256-byte aligned tables after the header)."""
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    words = plan.view(torch.int32).cpu().numpy()
    max_chunks = e // 65 + e // 1024 + 1
    off_light = 256
    off_chunks = al(off_light + n * 16)
    off_heavy = al(off_chunks + max_chunks * 16)
    hdr = words[:12]
    light = words[off_light // 4: off_light // 4 + 4 * hdr[0]].reshape(-1, 4)
    chunks = words[off_chunks // 4: off_chunks // 4 + 4 * hdr[1]].reshape(-1, 4)
    heavy = words[off_heavy // 4: off_heavy // 4 + 4 * hdr[2]].reshape(-1, 4)
    return hdr, light, chunks, heavy


def _plan_check(plan, n, e, rp):
    """The plan's header counts and every entry of its tables, from the row lengths: rows of
    at most 64 edges in the light list, longer rows cut into 1024-edge chunks, rows of more
    than one chunk in the heavy list with consecutive partial-state slots."""
    hdr, light, chunks, heavy = _plan_tables(plan, n, e)
    deg = np.diff(rp)
    nchunk = np.where(deg > 64, (deg + 1023) // 1024, 0)
    assert hdr[0] == (deg <= 64).sum()
    assert hdr[1] == nchunk.sum()
    assert hdr[2] == (nchunk > 1).sum()
    assert hdr[3] == nchunk[nchunk > 1].sum()
    assert hdr[4] == n and hdr[9] == e and hdr[10] == 0 and hdr[11] == 0
    assert hdr[8] == deg[deg <= 64].sum()  # edges of the light rows
    lv = np.nonzero(deg <= 64)[0]
    np.testing.assert_array_equal(light, np.stack([lv, rp[lv], rp[lv + 1], np.zeros_like(lv)], 1))
    cv = np.nonzero(deg > 64)[0]
    k = nchunk[cv]
    v = np.repeat(cv, k)
    j = np.arange(v.size) - np.repeat(np.cumsum(k) - k, k)
    cb = rp[v] + 1024 * j
    hv = cv[k > 1]
    first = np.cumsum(nchunk[hv]) - nchunk[hv]  # each heavy row's first slot
    slot_of = np.full(n, -1, np.int64)
    slot_of[hv] = first
    slot = np.where(nchunk[v] > 1, slot_of[v] + j, -1)
    np.testing.assert_array_equal(chunks, np.stack([v, cb, np.minimum(cb + 1024, rp[v + 1]), slot], 1).reshape(-1, 4))
    np.testing.assert_array_equal(heavy, np.stack([hv, first, nchunk[hv], np.zeros_like(hv)], 1).reshape(-1, 4))


@pytest.mark.parametrize("n", [1, 4095, 4096, 4097, 6000, 70_000])
def test_plan_counts(g, n):
    """The plan's tables follow from the degree histogram (node counts around the scan's
    4096-row blocks)."""
    hubs = (50000, 4097, 1025, 1024, 700, 65, 64) if n > 8 else ()
    src, dst = synth.mixed_degree_graph(n, 2, hubs=hubs, isolated=3 if n > 8 else 0)
    e = int(src.size)
    t = g.Topology(n, i32(src), i32(dst))
    torch.cuda.synchronize()
    rp = np.concatenate([[0], np.cumsum(np.bincount(dst, minlength=n))])
    _plan_check(t.plan, n, e, rp)


def test_plan_guard(g):
    """A plan is used only for the n and e it was built for, from a row_ptr consistent with
    e: otherwise the attention kernels process no row and write nothing (their outputs keep
    what they held) and gga_plan_status reports it; a correct call afterwards still works."""
    n, heads, c = 3000, 2, 16
    src, dst = synth.mixed_degree_graph(n, 3, hubs=(5000, 1500, 100))
    e = src.size
    topo = g.Topology(n, i32(src), i32(dst), backward=True)
    assert int(g.gga_plan_status(topo.plan, n, e).item()) == g.GGA_OK
    assert int(g.gga_plan_status(topo.plan, n, e - 1).item()) == g.GGA_EINVAL
    assert int(g.gga_plan_status(topo.plan, n + 1, e).item()) == g.GGA_EINVAL
    rng = np.random.default_rng(4)
    q, k, v = (torch.from_numpy(rng.standard_normal((n, heads, c)).astype(np.float32)).cuda() for _ in range(3))
    good = g.make_desc(n, e, heads, c, g.GGA_SCORE_DOT, g.GGA_F32)
    ref, ref_lse = g.gga_local_attn_fwd(good, q, k, v, topo.row_ptr, topo.col, topo.plan)
    torch.cuda.synchronize()
    # a plan built for e edges, handed a call over e - 7
    wrong = g.make_desc(n, e - 7, heads, c, g.GGA_SCORE_DOT, g.GGA_F32)
    out = torch.full((n, heads, c), 7.0, device="cuda")
    lse = torch.full((n, heads), 7.0, device="cuda")
    g.gga_local_attn_fwd(wrong, q, k, v, topo.row_ptr, topo.col, topo.plan, out=out, lse=lse)
    d_out = torch.ones_like(out)
    dq, dk, dv = (torch.full((n, heads, c), 7.0, device="cuda") for _ in range(3))
    g.gga_local_attn_bwd(wrong, q, k, v, ref, ref_lse, d_out, topo, d_qs=dq, d_ks=dk, d_v=dv)
    torch.cuda.synchronize()
    for t in (out, lse, dq, dk, dv):
        assert bool((t == 7.0).all())
    assert int(g.gga_plan_status(topo.plan, n, e).item()) == g.GGA_EINVAL  # misuse recorded
    again, again_lse = g.gga_local_attn_fwd(good, q, k, v, topo.row_ptr, topo.col, topo.plan)
    torch.cuda.synchronize()
    assert torch.equal(again, ref) and torch.equal(again_lse, ref_lse)
    # a row_ptr whose rows run past e: the plan is marked invalid at build time
    short = e - 100
    bad_plan = g.gga_plan_build(n, short, topo.row_ptr)
    assert int(g.gga_plan_status(bad_plan, n, short).item()) == g.GGA_ERANGE
    d_short = g.make_desc(n, short, heads, c, g.GGA_SCORE_DOT, g.GGA_F32)
    out.fill_(7.0)
    g.gga_local_attn_fwd(d_short, q, k, v, topo.row_ptr, topo.col, bad_plan, out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    # rows that overlap (row_ptr not monotone)
    rp = i32(np.array([0, 100, 50, 150], np.int32))
    assert int(g.gga_plan_status(g.gga_plan_build(3, 150, rp), 3, 150).item()) == g.GGA_ERANGE


def test_plan_corrupt_row_ptr(g):
    """A row_ptr with 1100 entries set near INT32_MAX: the rows before them claim about 2^21
    chunks each, so the chunk counts add up past 2^31 in the 32-bit scans.  Every table
    position is checked at both ends before it is written; the plan reports GGA_ERANGE and
    a forward handed it writes nothing."""
    n, e, heads, c = 4096, 300_000, 2, 16
    rng = np.random.default_rng(0)
    deg = rng.integers(0, 2 * e // n, n)
    deg = (deg * (e / deg.sum())).astype(np.int64)
    deg[-1] += e - deg.sum()
    rp = np.concatenate([[0], np.cumsum(deg)]).astype(np.int64)
    rp[rng.choice(np.arange(1, n), 1100, replace=False)] = np.iinfo(np.int32).max - 1
    print(f"plan over a corrupt row_ptr: n={n} e={e}", flush=True)
    plan = g.gga_plan_build(n, e, i32(rp))
    torch.cuda.synchronize()
    assert int(g.gga_plan_status(plan, n, e).item()) == g.GGA_ERANGE
    # the edges themselves are valid: a forward over them with this plan leaves its outputs
    col = i32(rng.integers(0, n, e))
    q, k, v = (torch.from_numpy(rng.standard_normal((n, heads, c)).astype(np.float32)).cuda() for _ in range(3))
    desc = g.make_desc(n, e, heads, c, g.GGA_SCORE_DOT, g.GGA_F32)
    out = torch.full((n, heads, c), 7.0, device="cuda")
    lse = torch.full((n, heads), 7.0, device="cuda")
    g.gga_local_attn_fwd(desc, q, k, v, i32(rp), col, plan, out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())


# ---- the largest inputs the boundary takes (e < INT32_MAX; n up to INT32_MAX - 1)


def _csr_properties(n, e, key, other, rp, col, eid, chunk=1 << 28):
    """The unique stable CSR, checked through properties that hold at any size: row_ptr
    runs from 0 to e without decreasing; every position lies in the row of its edge's key;
    col is the other endpoint of that edge; eid is a permutation of [0, e) that ascends
    within each row."""
    rp64 = rp.long()
    assert rp64[0].item() == 0 and rp64[-1].item() == e
    assert bool((rp64[1:] >= rp64[:-1]).all())
    seen = torch.zeros(e, dtype=torch.bool, device=key.device)
    prev_key = prev_id = None
    for p0 in range(0, e, chunk):
        p1 = min(e, p0 + chunk)
        ids = eid[p0:p1].long()
        assert bool(((ids >= 0) & (ids < e)).all())
        seen[ids] = True
        k = key[ids].long()
        pos = torch.arange(p0, p1, dtype=torch.long, device=key.device)
        assert bool(((rp64[k] <= pos) & (pos < rp64[k + 1])).all())
        assert bool((col[p0:p1] == other[ids]).all())
        same = k[1:] == k[:-1]
        assert bool((ids[1:][same] > ids[:-1][same]).all())
        if prev_key is not None and k[0].item() == prev_key:
            assert ids[0].item() > prev_id
        prev_key, prev_id = k[-1].item(), ids[-1].item()
        del ids, k, pos, same
    assert bool(seen.all())


@pytest.mark.timeout(900)
def test_csr_max_edges(g):
    # 2^31 - 2 edges over 2^21 rows: positions, COO indices and row_ptr values up to the
    # largest int32 the boundary accepts
    n, e = 1 << 21, (1 << 31) - 2
    gen = torch.Generator(device="cuda").manual_seed(7)
    key = torch.randint(0, n, (e,), generator=gen, dtype=torch.int32, device="cuda")
    other = torch.randint(0, n, (e,), generator=gen, dtype=torch.int32, device="cuda")
    print(f"csr at the largest edge count: n={n} e={e}", flush=True)
    rp, col, eid = g.gga_coo_to_csr(n, key, other)
    torch.cuda.synchronize()
    _csr_properties(n, e, key, other, rp, col, eid)
    del key, other, col, eid
    # the degree plan over the same row_ptr (rows of about 1024 edges: one or two chunks)
    print(f"plan at the largest edge count: n={n} e={e}", flush=True)
    plan = g.gga_plan_build(n, e, rp)
    torch.cuda.synchronize()
    _plan_check(plan, n, e, rp.cpu().numpy().astype(np.int64))
    del rp, plan
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_csr_max_rows(g):
    # 2^31 - 2 rows (31-bit keys: five passes) and 2^20 edges, bit-exact against the oracle
    n, e = (1 << 31) - 2, 1 << 20
    rng = np.random.default_rng(8)
    key = rng.integers(0, n, e, dtype=np.int64).astype(np.int32)
    key[:4] = (0, n - 1, n - 1, 0)
    other = rng.integers(0, n, e, dtype=np.int64).astype(np.int32)
    print(f"csr at the largest row count: n={n} e={e}", flush=True)
    rp, col, eid = g.gga_coo_to_csr(n, i32(key), i32(other))
    torch.cuda.synchronize()
    ref = oracle.coo_to_csr(n, key, other)
    np.testing.assert_array_equal(eid.cpu().numpy(), ref[2])
    np.testing.assert_array_equal(col.cpu().numpy(), ref[1])
    assert torch.equal(rp, torch.from_numpy(ref[0]).to(rp.device))
    del rp, col, eid, ref
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_edge_values_bwd_max_edges(g):
    # the endpoint projection's backward walks the CSR keyed by the endpoint with 64-bit
    # positions: the last row ends at 2^31 - 2, where a 32-bit step past it would wrap
    n, e = 1 << 21, (1 << 31) - 2
    gen = torch.Generator(device="cuda").manual_seed(9)
    key = torch.randint(0, n, (e,), generator=gen, dtype=torch.int32, device="cuda")
    print(f"edge_values_bwd at the largest edge count: n={n} e={e}", flush=True)
    rp, _, eid = g.gga_coo_to_csr(n, key, key)
    d_edge = torch.rand(e, 1, generator=gen, device="cuda")
    dx = g.gga_edge_values_bwd(n, d_edge, rp, eid)
    torch.cuda.synchronize()
    del eid
    ref = torch.zeros(n, dtype=torch.float64, device="cuda")
    chunk = 1 << 28
    for p0 in range(0, e, chunk):
        p1 = min(e, p0 + chunk)
        ref.index_add_(0, key[p0:p1].long(), d_edge[p0:p1, 0].double())
    deg = (rp[1:] - rp[:-1]).double()
    # fp32 sums of deg terms: rtol 1e-4 and atol 1e-5 sqrt(deg) (sums over long axes)
    err = (dx[:, 0].double() - ref).abs()
    assert bool((err <= 1e-4 * ref.abs() + 1e-5 * deg.clamp(min=1.0).sqrt()).all()), float(err.max())
    del key, rp, d_edge, dx, ref, deg, err
    torch.cuda.empty_cache()
