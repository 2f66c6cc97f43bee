"""Seeded synthetic inputs for the graph-attention workloads.

This module only draws random numbers and lays them out: graphs as int32 COO
edge lists (src = u, the key/value provider; dst = v, the query and the
softmax group), node tensors as float32 arrays, and bf16 copies made by
round-to-nearest-even.  It computes nothing of the attention method itself, so
both the CPU oracle and the GPU path can take their inputs from here.

Seeds follow one scheme: ``SeedSequence([workload_id, stream, *extra])`` with
stream 0 = topology, 1 = node tensors, 2 = weights, 3 = upstream gradients.
Large normal tensors are drawn in fixed chunks of 2**24 values, each chunk from
its own child seed, so the values do not depend on how many threads draw them.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

CHUNK = 1 << 24

TOPOLOGY, NODES, WEIGHTS, GRADS = 0, 1, 2, 3


def _rng(*parts: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(parts)))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(count: int, *seed: int, std: float = 1.0) -> np.ndarray:
    """``count`` float32 draws from N(0, std**2), chunked and seeded by ``seed``."""
    out = np.empty(count, np.float32)
    nch = (count + CHUNK - 1) // CHUNK

    def fill(i: int) -> None:
        a = i * CHUNK
        b = min(count, a + CHUNK)
        _rng(*seed, i).standard_normal(b - a, dtype=np.float32, out=out[a:b])

    if nch <= 1:
        if count:
            fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nch)))
    if std != 1.0:
        out *= np.float32(std)
    return out


def uniform_f32(count: int, lo: float, hi: float, *seed: int) -> np.ndarray:
    return _rng(*seed).uniform(lo, hi, count).astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """The exact float32 value of each bfloat16 bit pattern."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------- graphs


def _shuffle(src: np.ndarray, dst: np.ndarray, rng: np.random.Generator):
    perm = rng.permutation(src.shape[0])
    return np.ascontiguousarray(src[perm]), np.ascontiguousarray(dst[perm])


def _with_self_loops(src: np.ndarray, dst: np.ndarray, n: int):
    loops = np.arange(n, dtype=np.int32)
    return np.concatenate([src.astype(np.int32), loops]), np.concatenate([dst.astype(np.int32), loops])


def erdos_renyi(n: int, p: float, rng: np.random.Generator, self_loops: bool = True):
    """Directed Erdos-Renyi: each ordered pair u != v kept with probability p."""
    keep = rng.random((n, n)) < p  # keep[v, u]: edge u -> v
    np.fill_diagonal(keep, False)
    dst, src = np.nonzero(keep)
    src, dst = src.astype(np.int32), dst.astype(np.int32)
    if self_loops:
        src, dst = _with_self_loops(src, dst, n)
    return _shuffle(src, dst, rng)


def fixed_in_degree(n: int, k: int, rng: np.random.Generator, self_loops: bool = True):
    """Every destination gets exactly k sources drawn uniformly with replacement."""
    dst = np.repeat(np.arange(n, dtype=np.int32), k)
    src = rng.integers(0, n, size=n * k, dtype=np.int32)
    if self_loops:
        src, dst = _with_self_loops(src, dst, n)
    return _shuffle(src, dst, rng)


def uniform_pairs(n: int, m: int, rng: np.random.Generator, self_loops: bool = True):
    """m (src, dst) pairs drawn uniformly and independently."""
    src = rng.integers(0, n, size=m, dtype=np.int32)
    dst = rng.integers(0, n, size=m, dtype=np.int32)
    if self_loops:
        src, dst = _with_self_loops(src, dst, n)
    return _shuffle(src, dst, rng)


def pareto_in_degrees(n: int, mean: float, tail: float, cap: int, rng: np.random.Generator) -> np.ndarray:
    """In-degrees min(cap, floor(x_min * (1-U)**(-1/tail))) with x_min bisected so the
    realised mean is as close to ``mean`` as the floor allows (Zipf exponent tail+1)."""
    base = (1.0 - rng.random(n)) ** (-1.0 / tail)

    def realised(xm: float) -> float:
        return float(np.minimum(cap, np.floor(xm * base)).mean())

    lo, hi = 0.0, 1.0
    while realised(hi) < mean:
        hi *= 2.0
    for _ in range(100):
        mid = 0.5 * (lo + hi)
        if realised(mid) < mean:
            lo = mid
        else:
            hi = mid
    return np.minimum(cap, np.floor(hi * base)).astype(np.int64)


def power_law(n: int, mean: float, tail: float, cap: int, rng: np.random.Generator, self_loops: bool = True):
    deg = pareto_in_degrees(n, mean, tail, cap, rng)
    dst = np.repeat(np.arange(n, dtype=np.int32), deg)
    src = rng.integers(0, n, size=dst.shape[0], dtype=np.int32)
    if self_loops:
        src, dst = _with_self_loops(src, dst, n)
    return _shuffle(src, dst, rng)


def random_multigraph(n: int, m: int, seed: int, self_loops: bool = True, isolated: int = 0):
    """Small test graphs: m uniform pairs (duplicates allowed), optional self-loops,
    and the last ``isolated`` nodes given no in-edges at all."""
    rng = _rng(9000, seed)
    live = max(1, n - isolated)
    src = rng.integers(0, n, size=m, dtype=np.int32)
    dst = rng.integers(0, live, size=m, dtype=np.int32)
    if self_loops:
        loops = np.arange(live, dtype=np.int32)
        src = np.concatenate([src, loops])
        dst = np.concatenate([dst, loops])
    if n == 0:
        return np.zeros(0, np.int32), np.zeros(0, np.int32)
    return _shuffle(src, dst, rng)


# --------------------------------------------------------------------------- workloads


@dataclass(frozen=True)
class Workload:
    ident: int
    name: str
    n: int
    heads: int
    head_dim: int
    dtype: str  # storage type of the node tensors: "f32" or "bf16"
    score: str  # "dot" or "additive"
    fin: int = 0  # GAT input width
    d_model: int = 0  # gated layer model width
    batch: int = 1  # graphs packed along the node axis (n nodes in all)
    relations: int = 0  # relation types of the edges (relation-typed messages)


WORKLOADS = {
    1: Workload(1, "tiny-dot-er-n1024", 1024, 1, 16, "f32", "dot"),
    2: Workload(2, "gat-powerlaw-n170k", 170_000, 8, 8, "f32", "additive", fin=128),
    3: Workload(3, "dot-uniform16-n1m-h8-r64-bf16", 1 << 20, 8, 64, "bf16", "dot"),
    4: Workload(4, "gated-layer-n262k-d256-h4", 1 << 18, 4, 64, "f32", "dot", d_model=256),
    5: Workload(5, "dot-zipf1.8-n2m-h8-c32-bf16", 1 << 21, 8, 32, "bf16", "dot"),
    6: Workload(6, "gated-layer-batch64-n4096-d256-h4", 1 << 18, 4, 64, "f32", "dot", d_model=256, batch=64),
    7: Workload(7, "gat-edgefeat-mean-powerlaw-n170k", 170_000, 8, 8, "f32", "additive", fin=128),
    8: Workload(8, "relation-mean-packed-512x256-d512-h8-r3", 512 * 256, 8, 64, "f32", "mean", d_model=512,
                batch=512, relations=3),
    9: Workload(9, "relation-softmax-packed-512x256-d512-h8-r3", 512 * 256, 8, 64, "f32", "dot", d_model=512,
                batch=512, relations=3),
}


def workload_graph(ident: int, n: int | None = None):
    """The COO edge list (src, dst) of a workload, optionally at a smaller node count
    with the same degree recipe.  Returns int32 arrays, shuffled into random COO order."""
    w = WORKLOADS[ident]
    n = w.n if n is None else n
    rng = _rng(ident, TOPOLOGY)
    if ident == 1:
        return erdos_renyi(n, 8.0 / (n - 1), rng)
    if ident in (2, 7):  # the edge-feature variant runs on the same graph
        return power_law(n, 14.0, 1.1, 10_000, _rng(2, TOPOLOGY))
    if ident == 3:
        return fixed_in_degree(n, 16, rng)
    if ident == 4:
        return uniform_pairs(n, 32 * n, rng)
    if ident == 5:
        return power_law(n, 31.0, 0.8, 50_000, rng)
    raise KeyError(ident)


def batch_of_graphs(sizes, degree: int, rng: np.random.Generator):
    """A batch of graphs, one adjacency list each: graph b has sizes[b] nodes, degree * n_b
    uniform (src, dst) pairs over its own nodes (duplicates allowed) plus one self-loop per
    node, shuffled within the graph.  Returns node_ptr [B+1], edge_ptr [B+1] and the local
    COO lists of all graphs, concatenated (int32)."""
    sizes = [int(x) for x in sizes]
    node_ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    srcs, dsts, counts = [], [], []
    for nb in sizes:
        s, d = uniform_pairs(nb, degree * nb, rng) if nb > 0 else (np.zeros(0, np.int32), np.zeros(0, np.int32))
        srcs.append(s)
        dsts.append(d)
        counts.append(s.shape[0])
    edge_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return node_ptr, edge_ptr, np.concatenate(srcs).astype(np.int32), np.concatenate(dsts).astype(np.int32)


def workload_batch(ident: int):
    """The per-graph COO lists of a batched workload (equal graph sizes n / batch)."""
    w = WORKLOADS[ident]
    return batch_of_graphs([w.n // w.batch] * w.batch, 32, _rng(ident, TOPOLOGY))


def relation_edges(sizes, degree: int, n_rel: int, rng: np.random.Generator):
    """Packed relation-typed edges over a batch of sequences (GiGL pull request "Support
    relation message modes on the packed GraphTransformerEncoder path": packed tokens,
    relation edges as rows (target, source, relation) with host-side (relation, start,
    end) segments).  Sequence b holds sizes[b] tokens; its edges are degree * n_b uniform
    (source, target) pairs over its own tokens plus one self-loop per token, each with a
    uniform relation in [0, n_rel).  The rows are grouped by relation (stable).  Returns
    n, src, dst (global packed ids, int32), rel and the segments [(r, start, end)]."""
    node_ptr, edge_ptr, sl, dl = batch_of_graphs(sizes, degree, rng)
    owner = np.repeat(np.arange(len(sizes)), np.diff(edge_ptr))
    src = (sl + node_ptr[owner]).astype(np.int32)
    dst = (dl + node_ptr[owner]).astype(np.int32)
    rel = rng.integers(0, n_rel, src.size).astype(np.int32)
    order = np.argsort(rel, kind="stable")
    src, dst, rel = src[order], dst[order], rel[order]
    bounds = np.searchsorted(rel, np.arange(n_rel + 1))
    segments = [(r, int(bounds[r]), int(bounds[r + 1])) for r in range(n_rel)]
    return int(node_ptr[-1]), src, dst, rel, segments


def workload_relation_edges(ident: int):
    """Relation workloads: sequences of n / batch tokens, 8 uniform in-edges per token plus
    a self-loop, uniform relations."""
    w = WORKLOADS[ident]
    return relation_edges([w.n // w.batch] * w.batch, 8, w.relations, _rng(8, TOPOLOGY))


def relation_inputs(n: int, d: int, heads: int, ch: int, n_rel: int, ident: int = 8):
    """X ~ N(0,1) [n,d]; W_Q [d, H*C] and the per-relation W_K, W_V [R, d, H*C] ~ N(0, 1/d),
    so that projected rows have unit scale; upstream gradient ~ N(0,1) [n, H*C]."""
    w = heads * ch
    x = node_tensor(ident, 0, (n, d))
    std = d ** -0.5
    w_q = normal_f32(d * w, ident, WEIGHTS, 0, std=std).reshape(d, w)
    w_k = normal_f32(n_rel * d * w, ident, WEIGHTS, 1, std=std).reshape(n_rel, d, w)
    w_v = normal_f32(n_rel * d * w, ident, WEIGHTS, 2, std=std).reshape(n_rel, d, w)
    d_out = node_tensor(ident, 0, (n, w), stream=GRADS)
    return dict(x=x, w_q=w_q, w_k=w_k, w_v=w_v, d_out=d_out)


def ragged_batch(seed: int, sizes=(1, 0, 17, 300, 4096, 2, 1000, 0, 2500, 63)):
    """Test batch with graphs of very different sizes, including empty ones."""
    return batch_of_graphs(sizes, 8, _rng(9200, seed))


def node_tensor(ident: int, which: int, shape, stream: int = NODES, std: float = 1.0) -> np.ndarray:
    count = int(np.prod(shape))
    return normal_f32(count, ident, stream, which, std=std).reshape(shape)


def gat_inputs(n: int, fin: int = 128, heads: int = 8, ch: int = 8, ident: int = 2):
    """X ~ N(0,1) [n,fin]; W Glorot-uniform [fin, heads*ch]; a_s, a_t ~ N(0, 0.1^2) [heads, ch];
    upstream gradient dOut ~ N(0,1) [n, heads*ch]."""
    x = node_tensor(ident, 0, (n, fin))
    lim = float(np.sqrt(6.0 / (fin + heads * ch)))
    w = uniform_f32(fin * heads * ch, -lim, lim, ident, WEIGHTS, 0).reshape(fin, heads * ch)
    a_s = normal_f32(heads * ch, ident, WEIGHTS, 1, std=0.1).reshape(heads, ch)
    a_t = normal_f32(heads * ch, ident, WEIGHTS, 2, std=0.1).reshape(heads, ch)
    d_out = node_tensor(ident, 0, (n, heads * ch), stream=GRADS)
    return x, w, a_s, a_t, d_out


def gat_edge_inputs(e: int, fe: int = 16, heads: int = 8, ch: int = 8, ident: int = 7):
    """Learned edge features of the GAT score: F ~ N(0,1) [e, fe] (COO order), W_e
    Glorot-uniform [fe, heads*ch], a_e ~ N(0, 0.1^2) [heads, ch]."""
    f = normal_f32(e * fe, ident, NODES, 1).reshape(e, fe)
    lim = float(np.sqrt(6.0 / (fe + heads * ch)))
    w_e = uniform_f32(fe * heads * ch, -lim, lim, ident, WEIGHTS, 3).reshape(fe, heads * ch)
    a_e = normal_f32(heads * ch, ident, WEIGHTS, 4, std=0.1).reshape(heads, ch)
    return dict(f=f, w_e=w_e, a_e=a_e)


def gated_layer_inputs(n: int, d: int = 256, ident: int = 4):
    """X ~ N(0,1) [n,d]; W_Q, W_K, W_V, W_o ~ N(0, 0.02^2) [d,d]; w_g [d], b_g ~ N(0, 0.02^2);
    LayerNorm gamma = 1, beta = 0."""
    x = node_tensor(ident, 0, (n, d))
    ws = [normal_f32(d * d, ident, WEIGHTS, i, std=0.02).reshape(d, d) for i in range(4)]
    w_g = normal_f32(d, ident, WEIGHTS, 4, std=0.02)
    b_g = float(normal_f32(1, ident, WEIGHTS, 5, std=0.02)[0])
    gamma = np.ones(d, np.float32)
    beta = np.zeros(d, np.float32)
    return dict(x=x, w_q=ws[0], w_k=ws[1], w_v=ws[2], w_o=ws[3], w_g=w_g, b_g=b_g, gamma=gamma, beta=beta)


def mixed_degree_graph(n: int, seed: int, hubs=(3000, 1025, 700, 65), background: int = 4, isolated: int = 3):
    """Test graph exercising every degree bucket: a uniform background of about
    ``background`` in-edges per node plus a self-loop, nodes 0..len(hubs)-1 given the
    listed extra in-degrees, and the last ``isolated`` nodes left with no in-edge."""
    rng = _rng(9100, seed)
    live = n - isolated
    m = background * live
    src = [rng.integers(0, n, size=m, dtype=np.int32), np.arange(live, dtype=np.int32)]
    dst = [rng.integers(0, live, size=m, dtype=np.int32), np.arange(live, dtype=np.int32)]
    for i, d in enumerate(hubs):
        if i < live:
            src.append(rng.integers(0, n, size=d, dtype=np.int32))
            dst.append(np.full(d, i, np.int32))
    return _shuffle(np.concatenate(src), np.concatenate(dst), rng)
