"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (host code
only) and run over small graphs that reach every C entry point and the edge cases the
pages name (isolated rows, duplicate edges, self-loops, a hub split over many rows of the
other orientation, an empty graph, ids outside their graph, relation rows).  A sanitizer
report aborts the child process; its results must also equal the plain build's."""

import os
import subprocess
import sys

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Runs in a child process (the sanitizer runtimes are preloaded there) and in this one.
SCRIPT = r'''
import sys
import numpy as np
sys.path.insert(0, globals().get("ROOT_DIR") or sys.argv[1])
import oracle, synth

def run():
    res = {}
    rng = np.random.default_rng(5)
    n = 40
    src, dst = synth.random_multigraph(n, 300, 3, isolated=4)
    src = np.concatenate([src, np.full(90, 7, np.int32), [5, 5]]).astype(np.int32)  # a hub source, duplicates
    dst = np.concatenate([dst, rng.integers(0, n - 4, 90).astype(np.int32), [9, 9]]).astype(np.int32)
    g = oracle.Graph(n, src, dst)
    res["csr"] = np.concatenate([g.row_ptr, g.col, g.eid, g.row_ptr_s, g.col_s, g.eid_s])
    try:
        oracle.coo_to_csr(n, np.array([0, n], np.int32), np.array([0, 0], np.int32))
        res["range"] = np.array([0])
    except ValueError:
        res["range"] = np.array([1])
    for hh, c in ((2, 3), (1, 16)):
        q, k, v, d = (rng.standard_normal((n, hh, c)) for _ in range(4))
        o, l = oracle.local_fwd_dot(q, k, v, g, c ** -0.5)
        r = oracle.local_bwd_dot(q, k, v, d, g, c ** -0.5)
        rows = np.array([0, 3, n - 1, 9], np.int32)
        o2, _ = oracle.local_fwd_dot(q, k, v, g, c ** -0.5, rows=rows)
        r2 = oracle.local_bwd_dot(q, k, v, d, g, c ** -0.5, rows_d=rows, rows_s=rows)
        res[f"dot{hh}"] = np.concatenate([a.ravel() for a in (o, np.where(np.isinf(l), 0, l), r["d_q"], r["d_k"],
                                                              r["d_v"], o2, r2["d_q"], r2["d_k"], r2["d_v"])])
    hf, d = rng.standard_normal((n, 3, 4)), rng.standard_normal((n, 3, 4))
    ss, sd, se = rng.standard_normal((n, 3)), rng.standard_normal((n, 3)), rng.standard_normal((src.size, 3))
    o, l = oracle.local_fwd_add(ss, sd, hf, g, s_edge=se)
    r = oracle.local_bwd_add(ss, sd, hf, d, g, s_edge=se)
    res["add"] = np.concatenate([a.ravel() for a in (o, r["d_s_src"], r["d_s_dst"], r["d_hf"], r["d_s_edge"])])
    x = rng.standard_normal((n, 5))
    res["edge"] = np.concatenate([oracle.edge_values(x, src).ravel(),
                                  oracle.edge_values_bwd(rng.standard_normal((src.size, 5)), dst, n).ravel()])
    e0 = oracle.Graph(6, np.zeros(0, np.int32), np.zeros(0, np.int32))
    o, l = oracle.local_fwd_dot(np.ones((6, 1, 2)), np.ones((6, 1, 2)), np.ones((6, 1, 2)), e0, 1.0)
    res["empty"] = o.ravel()
    node_ptr = np.array([0, 3, 3, 10], np.int32)
    edge_ptr = np.array([0, 4, 4, 9], np.int32)
    sl = np.array([0, 1, 2, 3, 0, 6, 7, -1, 2], np.int32)
    dl = np.array([1, 2, 0, 0, 6, 0, 1, 2, 2], np.int32)
    bs, bd, bad = oracle.batch_edges(node_ptr, edge_ptr, sl, dl)
    res["batch"] = np.concatenate([bs, bd, [bad]])
    n_rel, heads, ch = 3, 2, 4
    rel = rng.integers(0, n_rel, src.size).astype(np.int32)
    xr = rng.standard_normal((n, 6))
    wq, wk, wv = rng.standard_normal((6, 8)), rng.standard_normal((n_rel, 6, 8)), rng.standard_normal((n_rel, 6, 8))
    dout = rng.standard_normal((n, 8))
    for mode in (oracle.REL_SOFTMAX, oracle.REL_MEAN):
        f = oracle.relation_forward(xr, wq, wk, wv, src, dst, rel, heads, mode)
        b = oracle.relation_backward(xr, wq, wk, wv, src, dst, rel, heads, mode, dout)
        res[f"rel{mode}"] = np.concatenate([f["out"].ravel(), b["d_x"].ravel(), b["d_w_v"].ravel()])
    return res

if __name__ == "__main__":
    np.savez(sys.argv[2], **run())
'''


def test_oracle_under_sanitizers(tmp_path):
    lib = oracle.build(force=True, path=str(tmp_path / "_oracle_san.so"), sanitize=True)
    script = tmp_path / "drive.py"
    script.write_text(SCRIPT)
    out = tmp_path / "san.npz"
    runtimes = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
        if not os.path.isabs(p):
            pytest.skip(f"{name} is not available")
        runtimes.append(p)
    # the sanitizer runtimes go first; whatever the environment already preloads stays after them
    preload = " ".join(runtimes + [p for p in [os.environ.get("LD_PRELOAD", "")] if p])
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=preload, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, str(script), ROOT, str(out)], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, f"sanitized oracle failed:\n{r.stderr[-4000:]}"
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
    san = np.load(out)
    ns = {"ROOT_DIR": ROOT}
    exec(compile(SCRIPT.replace('if __name__ == "__main__":', "if False:"), "drive", "exec"), ns)
    sys.path.insert(0, ROOT)
    plain = ns["run"]()
    assert set(plain) == set(san.files)
    for k in plain:
        np.testing.assert_allclose(san[k], plain[k], rtol=1e-12, atol=1e-12, err_msg=k)
