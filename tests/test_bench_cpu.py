"""Host-side checks of bench.py: the single-GPU contract, the algorithmic byte counts behind
the roofline (the forward's one key row, one value row and one column id per edge, the
target's q, out and lse once), and the roofline record."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr and r.stdout == ""


def test_forward_algorithmic_bytes():
    import bench

    n, e, heads, c = 1 << 20, 17 << 20, 8, 64  # the 1M-node workload: 16 uniform in-edges + a self-loop
    w = heads * c
    q, kv, col, row_ptr, out, lse = n * w * 2, e * 2 * w * 2, e * 4, 4 * (n + 1), n * w * 4, n * heads * 4
    assert bench.fwd_bytes(n, e, heads, c, 2) == q + kv + col + row_ptr + out + lse == 39_837_499_396
    # without lse: 39.80 GB, the figure the workload is specified with
    assert abs(bench.fwd_bytes(n, e, heads, c, 2, with_lse=False) / 1e9 - 39.80) < 0.005
    # the heavy-tailed 2M-node workload (E = 2^26 with self-loops, 8 heads of 32): 72.3 GB
    assert abs(bench.fwd_bytes(1 << 21, 1 << 26, 8, 32, 2) / 1e9 - 72.3) < 0.05


def test_backward_algorithmic_bytes():
    import bench

    n, e, heads, c, esz = 1 << 21, 1 << 26, 8, 32, 2
    w = heads * c
    # pass A, CSR by destination: a key and a value row and col per edge; q, dO, out, lse,
    # row_ptr read and dq, D written per node
    pass_a = e * (2 * w * esz + 4) + n * (w * esz + 4 * w + 4 * w + 4 * heads + 4) + n * (4 * w + 4 * heads)
    # pass B, CSR by source: per edge the target's q and dO rows, lse and D, and col; k, v,
    # row_ptr read and dk, dv written per node
    pass_b = e * (w * esz + 4 * w + 8 * heads + 4) + n * (2 * w * esz + 4) + n * 2 * 4 * w
    assert bench.bwd_bytes(n, e, heads, c, esz) == pass_a + pass_b == 190_740_168_704
    assert abs(pass_a / 1e9 - 76.6) < 0.05 and abs(pass_b / 1e9 - 114.1) < 0.05


def test_roofline_record():
    import bench

    r = bench.roofline("hbm", 5000.0, 8000.0, "GB/s", traffic=39.86, kernel="k")
    assert r == {"bound": "hbm", "achieved": 5000.0, "peak": 8000.0, "unit": "GB/s", "frac": 0.625,
                 "traffic": 39.86, "kernel": "k"}


def test_roofline_never_above_peak():
    import pytest

    import bench

    with pytest.raises(ValueError):
        bench.roofline("hbm", 8100.0, 8000.0, "GB/s")


def test_counted_traffic_is_tied_to_its_profile_and_sources():
    """Every counted figure names a committed profile summary that states it and the digest of
    the kernel sources it was taken with; a changed kernel reports no counted figure."""
    import bench

    for key, c in bench.COUNTED.items():
        if c["gb"] is None:
            assert bench.counted_traffic(key) is None
            continue
        txt = open(os.path.join(ROOT, c["profile"])).read()
        assert f"{c['gb']:.2f} GB" in txt, (key, c["profile"])
        assert c["digest"] in txt, (key, c["profile"])
        assert len(c["digest"]) == 16
        if c["digest"] == bench.sources_digest(c["sources"]):
            assert bench.counted_traffic(key) == c["gb"]
        else:
            assert bench.counted_traffic(key) is None
