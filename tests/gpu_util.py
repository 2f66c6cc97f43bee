"""Helpers for the GPU parity tests: seeded inputs on the device and on the host."""

import numpy as np
import torch

import oracle
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


def global_term_scales(q, k, v, d_g, eps, node_ptr=None):
    """Per element, the sum of the magnitudes of the terms each gradient of the global branch
    adds (S and dS taken as sums of |terms| over the nodes, since their own rounding error
    scales with those): an fp32 evaluation is off by at most a small multiple of 2^-24 times
    this, also where the terms cancel (one node: dq is only eps-sized)."""
    q, k, v, d_g = (np.asarray(a, np.float64) for a in (q, k, v, d_g))
    if node_ptr is not None:  # per graph of a batch
        out = {nm: np.zeros(q.shape) for nm in ("d_q", "d_k", "d_v")}
        for b in range(len(node_ptr) - 1):
            lo, hi = int(node_ptr[b]), int(node_ptr[b + 1])
            if hi > lo:
                one = global_term_scales(q[lo:hi], k[lo:hi], v[lo:hi], d_g[lo:hi], eps)
                for nm in out:
                    out[nm][lo:hi] = one[nm]
        return out
    t = lambda a: a.transpose(1, 0, 2)  # noqa: E731
    s, z, gg = oracle.global_linear(q, k, v, eps)
    pq, pk = oracle.phi(q), oracle.phi(k)
    s_abs = pk.transpose(1, 2, 0) @ t(np.abs(v))
    den = (pq * z[None]).sum(-1) + eps
    a_num = np.abs(d_g) / den[..., None]
    a_den = (np.abs(d_g) * np.abs(gg)).sum(-1) / den
    tq = (t(t(a_num) @ s_abs.transpose(0, 2, 1)) + z[None] * a_den[..., None]) * oracle.phi_grad(q)
    ds_abs = pq.transpose(1, 2, 0) @ t(a_num)
    dz_abs = (pq * a_den[..., None]).sum(0)
    tk = (t(t(np.abs(v)) @ ds_abs.transpose(0, 2, 1)) + dz_abs[None]) * oracle.phi_grad(k)
    tv = t(t(pk) @ ds_abs)
    return dict(d_q=tq, d_k=tk, d_v=tv)
