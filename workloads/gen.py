"""Seeded value generation for the workloads in ``configs.py``.

Draw order, from ``numpy.random.default_rng(seed)``: for every append in the
trace, in trace order, K then V as standard normals of shape [L][n][Hkv][D]
(float32); then the queries. bf16 values are the round-to-nearest-even
rounding of those float32 draws, kept as their raw 16-bit patterns; the
float32 copy consumers see is the exact upcast of the bf16 value. Draft-tree
parent pointers for verify workloads come from a per-request generator
``default_rng([seed, r])``.

Nothing here computes any part of the method: this is input preparation only.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .configs import Shape, Workload


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.
    Inputs are finite draws, so no NaN/Inf handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class Tensor:
    """A generated array in its storage type: ``raw`` is float32 for f32
    workloads and the uint16 bit pattern for bf16; ``f32()`` gives the exact
    float32 value either way."""

    __slots__ = ("raw", "dtype")

    def __init__(self, raw: np.ndarray, dtype: str):
        self.raw = raw
        self.dtype = dtype

    def f32(self) -> np.ndarray:
        return self.raw if self.dtype == "f32" else bf16_to_f32(self.raw)

    @property
    def shape(self):
        return self.raw.shape


def draw(rng: np.random.Generator, shape_tuple, dtype: str) -> Tensor:
    x = rng.standard_normal(shape_tuple, dtype=np.float32)
    if dtype == "f32":
        return Tensor(x, "f32")
    return Tensor(bf16_round(x), "bf16")


def draw_kv(rng: np.random.Generator, shape: Shape, n: int):
    """K then V for ``n`` new tokens, each [L][n][Hkv][D]."""
    k = draw(rng, (shape.L, n, shape.Hkv, shape.D), shape.dtype)
    v = draw(rng, (shape.L, n, shape.Hkv, shape.D), shape.dtype)
    return k, v


def verify_parents(seed: int, r: int, n_nodes: int, max_depth: int) -> np.ndarray:
    """Random best-first draft tree for request ``r``: node 0 hangs off the
    context (parent -1, depth 1); node i >= 1 picks its parent uniformly among
    the earlier nodes whose depth is below ``max_depth``. Parents therefore
    precede children, and no node is deeper than ``max_depth``."""
    rng = np.random.default_rng([seed, r])
    parent = np.full(n_nodes, -1, dtype=np.int32)
    depth = np.zeros(n_nodes, dtype=np.int64)
    if n_nodes:
        depth[0] = 1
    for i in range(1, n_nodes):
        cand = np.nonzero(depth[:i] < max_depth)[0]
        p = int(cand[rng.integers(len(cand))])
        parent[i] = p
        depth[i] = depth[p] + 1
    return parent


@dataclass
class Inputs:
    workload: Workload
    appends: List[tuple] = field(default_factory=list)   # (op index, sid, K Tensor, V Tensor)
    q: Optional[Tensor] = None      # decode: [L][B][Hq][D]; verify: [R][N][Hq][D]
    parents: Optional[np.ndarray] = None   # verify: int32 [R][N]


def generate(w: Workload, q_only: bool = False) -> Inputs:
    """All values for workload ``w``. With ``q_only`` the K/V draws are still
    made (to keep the stream aligned) but not kept."""
    sh = w.shape
    rng = np.random.default_rng(w.seed)
    inp = Inputs(w)
    for i, op in enumerate(w.ops):
        if op.kind != "append":
            continue
        k, v = draw_kv(rng, sh, op.n)
        if not q_only:
            inp.appends.append((i, op.sid, k, v))
    if w.kind == "decode":
        inp.q = draw(rng, (sh.L, len(w.query_sids), sh.Hq, sh.D), sh.dtype)
    else:
        inp.q = draw(rng, (len(w.query_sids), w.n_nodes, sh.Hq, sh.D), sh.dtype)
        inp.parents = np.stack([verify_parents(w.seed, r, w.n_nodes, w.max_depth)
                                for r in range(len(w.query_sids))]).astype(np.int32)
    return inp
