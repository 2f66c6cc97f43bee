"""Pins of the oracle's COO->CSR and endpoint projection against library routines.

The CSR by destination must equal a stable argsort of the destination column
(numpy, a library routine) and the histogram closed form; each row's edges keep
ascending COO index (Tinymesh "Sparse attention experiment", "Target softmax":
reductions walk the destination CSR, gathers keep COO order).
"""

import numpy as np
import pytest

import oracle
import synth


def _check_csr(n, key, other):
    row_ptr, col, eid = oracle.coo_to_csr(n, key, other)
    ref_eid = np.argsort(key, kind="stable").astype(np.int32)
    ref_ptr = np.concatenate([[0], np.cumsum(np.bincount(key, minlength=n))]).astype(np.int32)
    np.testing.assert_array_equal(row_ptr, ref_ptr)
    np.testing.assert_array_equal(eid, ref_eid)
    np.testing.assert_array_equal(col, other[ref_eid])
    # each row's eids ascend
    for v in range(n):
        seg = eid[row_ptr[v]:row_ptr[v + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(key[seg] == v)


@pytest.mark.parametrize("n,m,seed", [(1, 0, 0), (1, 5, 1), (7, 30, 2), (64, 500, 3), (300, 40, 4), (1000, 9000, 5)])
def test_csr_matches_stable_argsort(n, m, seed):
    src, dst = synth.random_multigraph(n, m, seed, self_loops=(seed % 2 == 0), isolated=n // 4)
    _check_csr(n, dst, src)
    _check_csr(n, src, dst)


def test_csr_empty_graph():
    row_ptr, col, eid = oracle.coo_to_csr(5, np.zeros(0, np.int32), np.zeros(0, np.int32))
    assert row_ptr.tolist() == [0] * 6 and col.size == 0 and eid.size == 0


def test_csr_hub_and_duplicates():
    n = 50
    src = np.array([3] * 20 + list(range(50)) + [7, 7, 7], np.int32)
    dst = np.array([9] * 20 + [9] * 50 + [9, 9, 9], np.int32)
    rng = np.random.default_rng(0)
    p = rng.permutation(src.size)
    _check_csr(n, dst[p], src[p])


def test_csr_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.coo_to_csr(3, np.array([0, 3], np.int32), np.array([0, 1], np.int32))


@pytest.mark.parametrize("w", [1, 3, 8])
def test_edge_values_matches_indexing(w):
    n, m = 40, 300
    src, dst = synth.random_multigraph(n, m, 11, isolated=5)
    x = np.random.default_rng(1).standard_normal((n, w))
    np.testing.assert_array_equal(oracle.edge_values(x, src), x[src])
    np.testing.assert_array_equal(oracle.edge_values(x, dst), x[dst])
    d_edge = np.random.default_rng(2).standard_normal((src.size, w))
    for ep in (src, dst):
        ref = np.zeros((n, w))
        np.add.at(ref, ep, d_edge)
        np.testing.assert_allclose(oracle.edge_values_bwd(d_edge, ep, n), ref, rtol=1e-13, atol=1e-13)


def test_edge_values_bwd_isolated_zero():
    d_edge = np.ones((3, 2))
    dx = oracle.edge_values_bwd(d_edge, np.array([1, 1, 1], np.int32), 4)
    np.testing.assert_array_equal(dx[[0, 2, 3]], 0.0)
    np.testing.assert_array_equal(dx[1], [3.0, 3.0])
