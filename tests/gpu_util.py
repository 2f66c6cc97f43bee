"""Helpers for the GPU parity tests: seeded inputs on the device and on the host."""

import numpy as np
import torch

import synth

TOL = {"f32": dict(rtol=1e-4, atol=1e-5), "bf16": dict(rtol=2e-2, atol=1e-5)}


def dev():
    return torch.device("cuda:0")


def node_pair(x32: np.ndarray, dtype: str):
    """(host float32 values, device tensor) of a node tensor stored as `dtype`; for
    bf16 the host values are the exact values of the rounded device bits."""
    if dtype == "bf16":
        bits = synth.to_bf16_bits(x32)
        host = synth.bf16_bits_to_f32(bits).reshape(x32.shape)
        t = torch.from_numpy(bits.view(np.int16).reshape(x32.shape)).to(dev()).view(torch.bfloat16)
        return host, t
    return x32, torch.from_numpy(np.ascontiguousarray(x32)).to(dev())


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def sample_rows(row_ptr: np.ndarray, k: int, seed: int):
    """k random rows plus the 8 longest rows and up to 4 empty rows."""
    n = row_ptr.shape[0] - 1
    deg = np.diff(row_ptr)
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(n, size=min(k, n), replace=False).tolist())
    rows.update(np.argsort(deg)[-8:].tolist())
    rows.update(np.nonzero(deg == 0)[0][:4].tolist())
    return np.array(sorted(rows), np.int32)


def assert_close(got, want, dtype: str, what: str, atol=None, rtol=None):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    tol = dict(TOL[dtype])
    if atol is not None:
        tol["atol"] = atol
    if rtol is not None:
        tol["rtol"] = rtol
    with np.errstate(invalid="ignore"):
        err = np.abs(got - want)
    lim = tol["atol"] + tol["rtol"] * np.abs(want)
    finite = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), finite), f"{what}: non-finite pattern differs"
    assert np.array_equal(got[~finite], want[~finite]), f"{what}: infinities differ"
    bad = (err > lim) & finite
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; max abs err "
                           f"{err[finite].max():.3e}")
    return float(err[finite].max()) if finite.any() else 0.0
