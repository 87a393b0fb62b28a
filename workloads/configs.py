"""Workload shapes and the operation traces that build each tree of sequences.

Every workload is a list of operations on a pool of fixed-size KV blocks:

* ``create(sid)``          -- a new, empty sequence;
* ``fork(parent, sid)``    -- a new sequence that starts as a shallow copy of
                              ``parent`` (the branching step of beam search,
                              MCTS and speculative trees);
* ``append(sid, n)``       -- ``n`` new tokens of K/V written at the end of
                              ``sid`` (their values are drawn by ``gen.py``);
* ``free(sid)``            -- the sequence is released.

followed by one attention call over ``query_sids``: a decode step (one query
per sequence) or, for ``kind == "verify"``, a draft-tree verify pass in which
the last ``n_nodes`` tokens of each request are the nodes of a draft tree.

The shapes restate the five workloads this library is measured on (a tiny
four-way fork, beam search, an MCTS tree, agents sharing a system prompt and
a speculative verify tree) plus two added cases: ``tiny_b`` (a root whose last
block is partly filled, so that every branch's first append copies it) and
``beam_cow`` (beam heads with a partly filled prompt tail, so that each of the
eight forks copies on write).
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import List, Optional, Tuple


@dataclass(frozen=True)
class Op:
    kind: str            # "create" | "fork" | "append" | "free"
    sid: int             # the sequence acted on (the child, for fork)
    parent: int = -1     # fork only
    n: int = 0           # append only


@dataclass(frozen=True)
class Shape:
    L: int               # layers of KV held by the pool
    Hq: int              # query heads
    Hkv: int             # KV heads; query head h reads KV head h // (Hq // Hkv)
    D: int               # head dimension
    BS: int              # tokens per block
    dtype: str           # "f32" or "bf16": storage type of q, K and V

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def token_kv_bytes(self) -> int:
        """Bytes of K plus V for one token of one layer, all KV heads."""
        return 2 * self.Hkv * self.D * self.elem_bytes


@dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    seed: int
    ops: Tuple[Op, ...]
    query_sids: Tuple[int, ...]
    kind: str = "decode"           # "decode" | "verify"
    n_nodes: int = 0               # verify: draft-tree nodes per request
    max_depth: int = 0             # verify: maximum node depth (root node = 1)
    scale: Optional[float] = None  # softmax scale; None means 1/sqrt(D)
    note: str = ""

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / (self.shape.D ** 0.5)

    def num_blocks_bound(self) -> int:
        """An upper bound on blocks ever allocated by the trace: every append
        of n tokens takes at most ceil(n / BS) + 1 blocks (one extra for a
        copy-on-write of a shared, partly filled tail)."""
        bs = self.shape.BS
        return sum(-(-op.n // bs) + 1 for op in self.ops if op.kind == "append")


# ----------------------------------------------------------------- builders

def star_trace(root_len: int, n_branches: int, branch_len: int,
               free_root_before_appends: bool) -> Tuple[List[Op], List[int]]:
    """A root prompt forked into ``n_branches`` branches, each of which appends
    ``branch_len`` private tokens. When the root stays alive during the
    appends, every branch sees the root's tail block shared and (if it is
    partly filled) copies it before writing."""
    ops = [Op("create", 0), Op("append", 0, n=root_len)]
    kids = list(range(1, n_branches + 1))
    for k in kids:
        ops.append(Op("fork", k, parent=0))
    if free_root_before_appends:
        ops.append(Op("free", 0))
    for k in kids:
        if branch_len:
            ops.append(Op("append", k, n=branch_len))
    if not free_root_before_appends:
        ops.append(Op("free", 0))
    return ops, kids


def binary_tree_trace(root_len: int, depth: int, edge_len: int) -> Tuple[List[Op], List[int]]:
    """Breadth-first growth of a binary tree: each node is forked twice, each
    child appends ``edge_len`` tokens, then the parent handle is freed, so
    only the leaves stay alive and a block of depth k is shared by
    2**(depth-k) leaves."""
    ops = [Op("create", 0), Op("append", 0, n=root_len)]
    level = [0]
    nxt = 1
    for _ in range(depth):
        new_level = []
        for p in level:
            for _c in range(2):
                ops.append(Op("fork", nxt, parent=p))
                ops.append(Op("append", nxt, n=edge_len))
                new_level.append(nxt)
                nxt += 1
            ops.append(Op("free", p))
        level = new_level
    return ops, level


def verify_trace(n_req: int, ctx_len: int, n_nodes: int) -> Tuple[List[Op], List[int]]:
    """Independent requests: each holds a paged context followed by the K/V
    of its draft-tree nodes (node j at position ctx_len + j)."""
    ops: List[Op] = []
    for r in range(n_req):
        ops.append(Op("create", r))
        ops.append(Op("append", r, n=ctx_len))
        ops.append(Op("append", r, n=n_nodes))
    return ops, list(range(n_req))


def _star(name, shape, seed, root_len, n_br, br_len, free_early, note=""):
    ops, q = star_trace(root_len, n_br, br_len, free_early)
    return Workload(name, shape, seed, tuple(ops), tuple(q), note=note)


def _mcts(name, shape, seed, root_len, depth, edge_len, note=""):
    ops, q = binary_tree_trace(root_len, depth, edge_len)
    return Workload(name, shape, seed, tuple(ops), tuple(q), note=note)


def _verify(name, shape, seed, n_req, ctx_len, n_nodes, max_depth, note=""):
    ops, q = verify_trace(n_req, ctx_len, n_nodes)
    return Workload(name, shape, seed, tuple(ops), tuple(q), kind="verify",
                    n_nodes=n_nodes, max_depth=max_depth, note=note)


TINY = Shape(L=1, Hq=4, Hkv=2, D=64, BS=16, dtype="f32")
BEAM = Shape(L=32, Hq=32, Hkv=8, D=128, BS=16, dtype="bf16")
AGENT = Shape(L=1, Hq=24, Hkv=4, D=256, BS=32, dtype="bf16")

WORKLOADS = {
    # 64-token root = 4 full blocks: the forks share whole blocks, and each
    # branch's 16 tokens go to a fresh block of its own (no copy).
    "tiny_a": _star("tiny_a", TINY, 0, 64, 4, 16, False,
                    "root 64 tokens (4 full blocks) forked 4 ways, +16 tokens each"),
    # 56-token root = 3 full blocks + 8/16: each branch's first append copies
    # the shared tail (8 slots), fills it, then opens a fresh block.
    "tiny_b": _star("tiny_b", TINY, 0, 56, 4, 16, False,
                    "root 56 tokens (3 full blocks + 8) forked 4 ways, +16 tokens each"),
    "beam": _star("beam", BEAM, 1, 2048, 8, 256, True,
                  "8 beams forked from a 2048-token prompt, 256 private tokens each, 32 layers"),
    "mcts": _mcts("mcts", BEAM, 2, 4096, 6, 32,
                  "4096-token root, binary tree of depth 6 (64 leaves), 32 tokens per edge, 32 layers"),
    "agent": _star("agent", AGENT, 3, 13312, 4, 32768, True,
                   "4 requests sharing a 13,312-token prefix, 32,768 private tokens each"),
    "verify": _verify("verify", AGENT, 4, 4, 32768, 48, 8,
                      "4 requests x (32,768-token context + 48-node draft tree, depth <= 8)"),
    # beam heads with a partly filled prompt tail (2056 = 128 blocks + 8):
    # the root stays alive while the 8 forks append one token each, so every
    # fork copies the 8 valid slots of the shared tail on write.
    "beam_cow": _star("beam_cow", BEAM, 5, 2056, 8, 1, False,
                      "2056-token prompt (last block 8/16) forked 8 ways, +1 token each"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(name: str, new_name: Optional[str] = None, seed: Optional[int] = None,
           shape: Optional[Shape] = None, **kw) -> Workload:
    """A smaller instance of a workload's structure, for parity tests the
    oracle finishes in seconds. ``kw`` are the builder's size parameters:
    star: root_len, n_branches, branch_len; mcts: root_len, depth, edge_len;
    verify: n_req, ctx_len, n_nodes, max_depth. ``shape`` overrides the shape
    (use ``dataclasses.replace``)."""
    base = WORKLOADS[name]
    sh = shape or base.shape
    sd = base.seed if seed is None else seed
    nm = new_name or f"{name}_scaled"
    if name in ("tiny_a", "tiny_b", "beam", "agent", "beam_cow"):
        defaults = {"tiny_a": (64, 4, 16, False), "tiny_b": (56, 4, 16, False),
                    "beam": (2048, 8, 256, True), "agent": (13312, 4, 32768, True),
                    "beam_cow": (2056, 8, 1, False)}[name]
        root_len = kw.get("root_len", defaults[0])
        n_br = kw.get("n_branches", defaults[1])
        br_len = kw.get("branch_len", defaults[2])
        free_early = kw.get("free_root_early", defaults[3])
        return _star(nm, sh, sd, root_len, n_br, br_len, free_early, base.note + " (scaled)")
    if name == "mcts":
        return _mcts(nm, sh, sd, kw.get("root_len", 4096), kw.get("depth", 6),
                     kw.get("edge_len", 32), base.note + " (scaled)")
    if name == "verify":
        return _verify(nm, sh, sd, kw.get("n_req", 4), kw.get("ctx_len", 32768),
                       kw.get("n_nodes", 48), kw.get("max_depth", 8), base.note + " (scaled)")
    raise KeyError(name)


def replace_shape(shape: Shape, **kw) -> Shape:
    return dataclasses.replace(shape, **kw)
