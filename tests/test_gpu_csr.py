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


def test_validate_coo(g):
    src = np.array([0, 1, 5, -1, 2], np.int32)
    dst = np.array([1, 7, 2, 0, 2], np.int32)
    bad = g.gga_validate_coo(5, i32(src), i32(dst))
    assert int(bad.item()) == 3
    bad = g.gga_validate_coo(8, i32(src), i32(dst))
    assert int(bad.item()) == 1


def test_plan_counts(g):
    """The plan's header counts follow from the degree histogram."""
    n = 6000
    src, dst = synth.mixed_degree_graph(n, 2, hubs=(50000, 4097, 1025, 1024, 700, 65, 64))
    t = g.Topology(n, i32(src), i32(dst))
    hdr = t.plan[:36].view(torch.int32).cpu().numpy()
    deg = np.bincount(dst, minlength=n)
    light = (deg <= 64).sum()
    chunks = np.where(deg > 64, (deg + 1023) // 1024, 0)
    assert hdr[0] == light
    assert hdr[1] == chunks.sum()
    assert hdr[2] == (chunks > 1).sum()
    assert hdr[3] == chunks[chunks > 1].sum()
    assert hdr[8] == deg[deg <= 64].sum()  # edges of the light rows
