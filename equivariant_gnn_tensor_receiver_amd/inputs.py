"""Seeded synthetic inputs: radius graphs, features, weights, cotangents.

This module is shared by the tests, the benchmark and the oracle checks.  It
holds none of the convolution's arithmetic (no radial basis, harmonics,
coupling tables or selection rules): it only draws positions and random
tensors and builds receiver-sorted CSR edge lists.  Shapes that depend on the
path count are passed in by the caller.

Recipe (one ``numpy.random.default_rng(seed)`` per workload, draws in this
order): positions U[0,1)^{N x 3}; x ~ N(0,1); W ~ N(0, 1/(K*C_in)) for the
fully connected weights [K][P][C_in][C_out], or N(0, 1/K) for the channel-wise
weights [K][P][C]; g_out ~ N(0,1); gg_pos ~ N(0,1).  bf16 workloads round x and W to bf16 (round to
nearest even) and use the exact bf16 values on both sides.

Graphs are directed radius graphs with cutoff c = 5 Angstrom, edges sorted by
receiver then sender, no self loops.  The "Tiny" workload places 64 nodes in a
6 Angstrom cube and keeps each receiver's 8 nearest senders (ties to the lower
index).  The others place N nodes in an open cube of side L, with L chosen so
that the number of directed edges is N * mean_degree (a threshold on the sorted
pair distances of the unit cube; then the graph is recomputed from the fp32
positions, so E can differ from the target by a pair or two).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

CUTOFF = 5.0


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    num_nodes: int
    mean_degree: int          # 0 = k-nearest cap (Tiny)
    channels: int
    lmax: int                 # irreps 0e+1o+..., SH lmax equal
    num_basis: int
    dtype: str                # "f32" or "bf16" for x and W
    passes: tuple
    knn_cap: int = 0
    box: float = 0.0          # fixed cube side (Tiny)
    channelwise: bool = False  # W[k, p, c] ("uvu") instead of W[k, p, ci, co]

    @property
    def irreps(self) -> str:
        return "+".join(f"{self.channels}x{l}{'e' if l % 2 == 0 else 'o'}"
                        for l in range(self.lmax + 1))

    @property
    def rows(self) -> int:
        return (self.lmax + 1) ** 2


WORKLOADS = {
    "tiny": Workload("tiny", 0, 64, 0, 8, 1, 8, "f32", ("fwd",), knn_cap=8, box=6.0),
    "molecular": Workload("molecular", 1, 4096, 32, 32, 2, 8, "f32", ("fwd", "bwd")),
    "wide_l": Workload("wide_l", 2, 16384, 64, 64, 3, 8, "bf16", ("fwd", "bwd")),
    "edge_scaling": Workload("edge_scaling", 3, 32768, 256, 32, 2, 8, "f32", ("fwd", "bwd")),
    "force": Workload("force", 4, 8192, 64, 128, 2, 16, "f32", ("fwd", "bwd", "dbwd")),
    # the Molecular graph and features with the channel-wise connection
    "molecular_uvu": Workload("molecular_uvu", 1, 4096, 32, 32, 2, 8, "f32", ("fwd", "bwd"), channelwise=True),
}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 values."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are exactly representable in bf16."""
    return (np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def edges_to_csr(num_nodes: int, senders: np.ndarray, receivers: np.ndarray):
    """Sort by (receiver, sender) and return (rowptr int32 [N+1], senders int32 [E])."""
    order = np.lexsort((senders, receivers))
    s = senders[order].astype(np.int32)
    v = receivers[order].astype(np.int64)
    counts = np.bincount(v, minlength=num_nodes)
    rowptr = np.zeros(num_nodes + 1, dtype=np.int64)
    np.cumsum(counts, out=rowptr[1:])
    return rowptr.astype(np.int32), s


def knn_capped_graph(pos: np.ndarray, cutoff: float, cap: int):
    """Each receiver keeps its `cap` nearest senders within `cutoff` (ties: lower id)."""
    p = pos.astype(np.float64)
    n = len(p)
    d = np.linalg.norm(p[:, None, :] - p[None, :, :], axis=-1)
    snd, rcv = [], []
    for v in range(n):
        cand = [s for s in range(n) if s != v and d[v, s] < cutoff]
        cand.sort(key=lambda s: (d[v, s], s))
        for s in cand[:cap]:
            snd.append(s)
            rcv.append(v)
    return edges_to_csr(n, np.array(snd, dtype=np.int64), np.array(rcv, dtype=np.int64))


def radius_graph(pos: np.ndarray, cutoff: float):
    """All directed pairs with |pos[s]-pos[v]| < cutoff, s != v."""
    from scipy.spatial import cKDTree

    p = pos.astype(np.float64)
    pairs = cKDTree(p).query_pairs(cutoff, output_type="ndarray")
    if len(pairs):
        dd = np.linalg.norm(p[pairs[:, 0]] - p[pairs[:, 1]], axis=-1)
        pairs = pairs[dd < cutoff]
    s = np.concatenate([pairs[:, 0], pairs[:, 1]]).astype(np.int64)
    v = np.concatenate([pairs[:, 1], pairs[:, 0]]).astype(np.int64)
    return edges_to_csr(len(p), s, v)


def box_for_degree(unit: np.ndarray, cutoff: float, mean_degree: int) -> float:
    """Cube side L so that the unit-cube positions scaled by L have N*deg directed edges."""
    from scipy.spatial import cKDTree

    n = len(unit)
    target_pairs = n * mean_degree // 2
    l_bulk = cutoff * (4.0 * math.pi * (n - 1) / (3.0 * mean_degree)) ** (1.0 / 3.0)
    tree = cKDTree(unit.astype(np.float64))
    rmax = cutoff / (0.9 * l_bulk)
    while True:
        pairs = tree.query_pairs(rmax, output_type="ndarray")
        if len(pairs) > target_pairs:
            break
        rmax *= 1.15
    u = unit.astype(np.float64)
    dist = np.sort(np.linalg.norm(u[pairs[:, 0]] - u[pairs[:, 1]], axis=-1))
    t = 0.5 * (dist[target_pairs - 1] + dist[target_pairs])
    return cutoff / t


def sample_receivers(num_nodes: int, count: int, seed: int) -> np.ndarray:
    """Seeded sample of receiver ids (sorted, unique) for checks at full size."""
    rng = np.random.default_rng(10_000 + seed)
    return np.sort(rng.choice(num_nodes, size=min(count, num_nodes), replace=False))


def make_graph(w: Workload):
    """Positions (fp32 [N,3]), rowptr (int32 [N+1]), senders (int32 [E]), box side, rng."""
    rng = np.random.default_rng(w.seed)
    unit = rng.random((w.num_nodes, 3))
    if w.knn_cap:
        L = w.box
        pos = (unit * L).astype(np.float32)
        rowptr, senders = knn_capped_graph(pos, CUTOFF, w.knn_cap)
    else:
        L = box_for_degree(unit, CUTOFF, w.mean_degree)
        pos = (unit * L).astype(np.float32)
        rowptr, senders = radius_graph(pos, CUTOFF)
    return pos, rowptr, senders, L, rng


def make_tensors(rng, num_nodes, rows_in, c_in, rows_out, c_out, num_basis, num_paths, dtype="f32",
                 channelwise=False, w_dtype=None):
    """x [N,rows_in,c_in], W [K,P,c_in,c_out] (or [K,P,c_in] channel-wise), g_out [N,rows_out,c_out], gg_pos [N,3].

    `dtype` is the storage type of x and, unless `w_dtype` is given, of W."""
    x = rng.standard_normal((num_nodes, rows_in, c_in), dtype=np.float32)
    if channelwise:
        W = (rng.standard_normal((num_basis, num_paths, c_in), dtype=np.float32)
             * np.float32(math.sqrt(1.0 / num_basis)))
    else:
        W = (rng.standard_normal((num_basis, num_paths, c_in, c_out), dtype=np.float32)
             * np.float32(math.sqrt(1.0 / (num_basis * c_in))))
    g_out = rng.standard_normal((num_nodes, rows_out, c_out), dtype=np.float32)
    gg_pos = rng.standard_normal((num_nodes, 3), dtype=np.float32)
    if dtype == "bf16":
        x = bf16_round(x)
    if (dtype if w_dtype is None else w_dtype) == "bf16":
        W = bf16_round(W)
    return dict(x=x, W=W.astype(np.float32), g_out=g_out, gg_pos=gg_pos)


def make_workload(name: str, num_paths: int):
    """Everything one workload needs, deterministic in its seed."""
    w = WORKLOADS[name]
    pos, rowptr, senders, L, rng = make_graph(w)
    t = make_tensors(rng, w.num_nodes, w.rows, w.channels, w.rows, w.channels,
                     w.num_basis, num_paths, w.dtype, channelwise=w.channelwise)
    return dict(workload=w, pos=pos, rowptr=rowptr, senders=senders, box=L, **t)


def random_graph(num_nodes: int, mean_degree: float, seed: int, box: float | None = None):
    """Small radius graph for parity tests: N nodes in a cube sized for ~mean_degree."""
    rng = np.random.default_rng(seed)
    unit = rng.random((num_nodes, 3))
    if box is None:
        box = CUTOFF * (4.0 * math.pi * num_nodes / (3.0 * max(mean_degree, 1e-3))) ** (1.0 / 3.0)
    pos = (unit * box).astype(np.float32)
    rowptr, senders = radius_graph(pos, CUTOFF)
    return pos, rowptr, senders, rng
