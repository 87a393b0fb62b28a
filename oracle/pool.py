"""Oracle block pool, block tables, fork, append with copy-on-write, free.

Test infrastructure (see the package docstring). Written for readability, not
speed: plain Python sets, lists and dicts.

Readings of the source pages used here (the pages describe the mechanism but
print no algorithm):

* Memory is paged in fixed-size blocks (Dendrite reply, vLLM comparison).
  A pool has ``num_blocks`` blocks of ``block_size`` token slots each.
* A fork is a shallow copy of the parent's block table: the child's table is
  a copy of the parent's list of block ids and every listed block gains one
  reference. No K/V is copied (same passage: "shallow pointer copy").
* A block that is being written may not be aliased (Dendrite reply, "Why
  Rust?"). So when a sequence appends to a partly filled last block whose
  count is above one, the writer first takes a fresh block, copies the
  valid slots into it, drops one reference from the old block and points its
  table at the copy. Later tokens then fill the copy and fresh blocks.
* Allocation takes the free block that comes first in ``alloc_order`` (by
  default the lowest free id), so two implementations that follow the same
  rule produce identical tables.
* An append is all or nothing: if the pool runs dry part-way, every change
  it made is undone and ``OOMError`` is raised.
* Appending zero tokens writes nothing and so copies nothing.
* Truncating a sequence to its first n tokens releases the references of
  the blocks that then hold none of its tokens; a kept, partly filled last
  block keeps its count (a later append copies it if it is shared).
* Committing a verified draft tree (Ferrite page, section 04: best-first
  trees verified in one pass; section 06: speculation never changes the
  text) keeps the accepted path: the request's last n_nodes tokens are the
  tree (node j at position len - n_nodes + j); the accepted nodes must form
  a chain from a root (each one's parent is the one before it, the first
  one's parent is -1). The sequence becomes the context followed by the
  accepted nodes' K/V in path order, exactly as if those tokens had been
  appended one after another: truncate to the context, then append them.
  Like an append, a commit is all or nothing: if the re-append runs out of
  blocks, the truncation is undone too and ``OOMError`` is raised. A batch
  of commits (one verify step over several requests) truncates every
  request first and then appends the kept paths in request order, all or
  nothing over the batch.
* Prompt cache (Ferrite page, section 07, and the "Agents" measurement: a
  conversation is snapshotted at turn boundaries, resumes from the longest
  match, a system prompt shared by several agents is computed once, and a
  conversation that loses its slot is parked). Read here as a cache of full
  blocks keyed by their exact token ids and by the entry of the block before
  them, so a chain of entries from the root spells a whole token prefix:
  - insert(sid, tokens) walks the sequence's full blocks among its first
    len(tokens) positions; a block whose key is present only refreshes that
    entry, a new key makes an entry that holds one reference on the
    sequence's block (the block outlives the sequence: it is parked).
  - match(tokens) makes a new sequence from the longest chain of entries
    whose tokens are a prefix of ``tokens`` (whole blocks only); each block
    gains a reference, as in a fork.
  - Every insert or match is one use: the entries it walks get a fresh
    stamp. The next entry to evict is, among entries with no child entry
    whose block only the cache holds, the one with the oldest stamp, the
    deepest first on a tie (a use stamps one chain, so stamp and depth
    single one entry out). Evicting drops the entry and its reference, and
    the block goes back to the free list.
  - An allocation that finds no free block evicts one entry first. An
    append checks up front that free blocks plus the entries that eviction
    could reach (entries whose whole subtree only the cache holds) cover
    what it needs; else OOMError and no change.
  - The cache holds at most ``cache_capacity`` entries (default: the pool's
    block count). An insert that finds it full evicts as above, never an
    entry this insert has walked; with nothing to evict it stops.
"""

from __future__ import annotations

import copy
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


class OOMError(Exception):
    """The pool has no free block for a required allocation."""


class InvalidError(Exception):
    """Unknown or already freed sequence, or a bad argument."""


class OraclePool:
    def __init__(self, num_blocks: int, block_size: int,
                 alloc_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise InvalidError("pool sizes must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        order = list(range(num_blocks)) if alloc_order is None else [int(b) for b in alloc_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidError("alloc_order must be a permutation of the block ids")
        self.rank = {b: i for i, b in enumerate(order)}
        self.free_blocks = set(range(num_blocks))
        self.ref = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        # materialised K/V: a list of (K, V) chunks, each [L][n][Hkv][D],
        # marked read-only; the sequence's logical K/V is their concatenation
        # along axis 1. Chunks are never modified, so sharing them between a
        # parent and a child is the same, by value, as a deep copy.
        self.mat: Dict[int, List[Tuple[np.ndarray, np.ndarray]]] = {}
        self._next_sid = 0
        self.cow_log: List[Tuple[int, int, int]] = []   # every (src, dst, n_valid)
        # prompt cache: entry id -> record; (parent entry id or -1, tokens) -> entry id
        self.cache_capacity = num_blocks
        self.entries: Dict[int, dict] = {}
        self.entry_of: Dict[Tuple[int, Tuple[int, ...]], int] = {}
        self._next_eid = 0
        self._clock = 0

    # ----------------------------------------------------------- internals
    def _alloc(self) -> int:
        if not self.free_blocks and not self._evict_one():
            raise OOMError("pool exhausted")
        b = min(self.free_blocks, key=self.rank.__getitem__)
        self.free_blocks.remove(b)
        self.ref[b] = 1
        return b

    def _check(self, sid: int) -> None:
        if sid not in self.tables:
            raise InvalidError(f"unknown or freed sequence {sid}")

    def _snapshot(self):
        return (set(self.free_blocks), list(self.ref), copy.deepcopy(self.tables),
                dict(self.lens), len(self.cow_log), copy.deepcopy(self.entries),
                dict(self.entry_of))

    def _restore(self, snap) -> None:
        self.free_blocks, self.ref, self.tables, self.lens, ncow, self.entries, self.entry_of = snap
        del self.cow_log[ncow:]

    # ----------------------------------------------------------- prompt cache
    def _children(self, eid: int) -> List[int]:
        return [e for e, r in self.entries.items() if r["parent"] == eid]

    def _victim(self, spare_stamp: Optional[int] = None) -> Optional[int]:
        """The entry eviction takes next, or None."""
        best = None
        for e, r in self.entries.items():
            if self._children(e) or self.ref[r["block"]] != 1 or r["stamp"] == spare_stamp:
                continue
            key = (r["stamp"], -r["depth"])
            if best is None or key < best[0]:
                best = (key, e)
        return None if best is None else best[1]

    def _drop_entry(self, eid: int) -> None:
        r = self.entries.pop(eid)
        del self.entry_of[(r["parent"], r["tokens"])]
        b = r["block"]
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free_blocks.add(b)

    def _evict_one(self, spare_stamp: Optional[int] = None) -> bool:
        e = self._victim(spare_stamp)
        if e is None:
            return False
        self._drop_entry(e)
        return True

    def evictable(self) -> int:
        """How many entries repeated eviction could remove now: those whose
        whole subtree of entries holds blocks only the cache holds."""
        def ok(e):
            return self.ref[self.entries[e]["block"]] == 1 and all(ok(c) for c in self._children(e))
        return sum(1 for e in self.entries if ok(e))

    def cache_insert(self, sid: int, tokens: Sequence[int]) -> int:
        """Cache the full blocks of ``sid`` among its first len(tokens)
        positions, ``tokens`` being their ids. Returns the new entry count."""
        self._check(sid)
        tokens = [int(t) for t in tokens]
        if len(tokens) > self.lens[sid]:
            raise InvalidError("more token ids than the sequence holds")
        bs = self.block_size
        self._clock += 1
        stamp = self._clock
        parent, added = -1, 0
        k = v = None
        for i in range(len(tokens) // bs):
            key = (parent, tuple(tokens[i * bs:(i + 1) * bs]))
            if key in self.entry_of:
                parent = self.entry_of[key]
                self.entries[parent]["stamp"] = stamp
                continue
            if len(self.entries) >= self.cache_capacity and not self._evict_one(stamp):
                break
            if k is None:
                k, v = self.kv(sid)
            b = self.tables[sid][i]
            eid = self._next_eid
            self._next_eid += 1
            depth = 1 if parent == -1 else self.entries[parent]["depth"] + 1
            kv = (np.array(k[:, i * bs:(i + 1) * bs], copy=True),
                  np.array(v[:, i * bs:(i + 1) * bs], copy=True))
            for a in kv:
                a.flags.writeable = False
            self.entries[eid] = {"parent": parent, "tokens": key[1], "block": b, "depth": depth,
                                 "stamp": stamp, "kv": kv}
            self.entry_of[key] = eid
            self.ref[b] += 1
            parent = eid
            added += 1
        return added

    def cache_match(self, tokens: Sequence[int], sid: Optional[int] = None) -> Tuple[int, int]:
        """A new sequence holding the longest cached chain of whole blocks
        that ``tokens`` starts with. Returns (sid, tokens matched)."""
        tokens = [int(t) for t in tokens]
        bs = self.block_size
        self._clock += 1
        stamp = self._clock
        chain, parent = [], -1
        for i in range(len(tokens) // bs):
            e = self.entry_of.get((parent, tuple(tokens[i * bs:(i + 1) * bs])))
            if e is None:
                break
            self.entries[e]["stamp"] = stamp
            chain.append(e)
            parent = e
        s = self.create(sid)
        for e in chain:
            b = self.entries[e]["block"]
            self.tables[s].append(b)
            self.ref[b] += 1
        self.lens[s] = len(chain) * bs
        self.mat[s] = [self.entries[e]["kv"] for e in chain]
        return s, len(chain) * bs

    def cache_clear(self) -> None:
        for e in list(self.entries):
            self._drop_entry(e)

    # ----------------------------------------------------------- verbs
    def create(self, sid: Optional[int] = None) -> int:
        if sid is None:
            sid = self._next_sid
        if sid in self.tables:
            raise InvalidError(f"sequence {sid} exists")
        self._next_sid = max(self._next_sid, sid + 1)
        self.tables[sid] = []
        self.lens[sid] = 0
        self.mat[sid] = []
        return sid

    def fork(self, parent: int, sid: Optional[int] = None) -> int:
        self._check(parent)
        child = self.create(sid)
        self.tables[child] = list(self.tables[parent])
        for b in self.tables[child]:
            self.ref[b] += 1
        self.lens[child] = self.lens[parent]
        self.mat[child] = list(self.mat[parent])
        return child

    def append(self, sid: int, k: np.ndarray, v: np.ndarray):
        """Append ``n = k.shape[1]`` tokens. Returns (slots, cow_ops): the slot
        (block * block_size + offset) of each new token in order, and the
        copy-on-write operations (src, dst, n_valid) taken."""
        self._check(sid)
        if k.shape != v.shape or k.ndim != 4:
            raise InvalidError("K and V must both be [L][n][Hkv][D]")
        n = k.shape[1]
        if n == 0:
            return [], []
        bs = self.block_size
        ln = self.lens[sid]
        copies = 1 if ln % bs and self.ref[self.tables[sid][-1]] > 1 else 0
        need = copies + (ln + n + bs - 1) // bs - (ln + bs - 1) // bs
        if need > len(self.free_blocks) and need > len(self.free_blocks) + self.evictable():
            raise OOMError("pool exhausted")
        snap = self._snapshot()
        try:
            table = self.tables[sid]
            cows = []
            r = self.lens[sid] % bs
            if r != 0 and self.ref[table[-1]] > 1:
                new_b = self._alloc()
                old_b = table[-1]
                self.ref[old_b] -= 1
                table[-1] = new_b
                cows.append((old_b, new_b, r))
            slots = []
            for _ in range(n):
                pos = self.lens[sid]
                if pos % bs == 0:
                    table.append(self._alloc())
                slots.append(table[pos // bs] * bs + pos % bs)
                self.lens[sid] = pos + 1
        except OOMError:
            self._restore(snap)
            raise
        kc = np.array(k, copy=True)
        vc = np.array(v, copy=True)
        kc.flags.writeable = False
        vc.flags.writeable = False
        self.mat[sid] = self.mat[sid] + [(kc, vc)]
        self.cow_log.extend(cows)
        return slots, cows

    def truncate(self, sid: int, n: int) -> None:
        """Keep the first ``n`` tokens of ``sid`` (0 <= n <= length)."""
        self._check(sid)
        if n < 0 or n > self.lens[sid]:
            raise InvalidError("truncate length outside [0, length]")
        bs = self.block_size
        keep = (n + bs - 1) // bs
        table = self.tables[sid]
        for b in table[keep:]:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free_blocks.add(b)
        del table[keep:]
        self.lens[sid] = n
        if n == 0:
            self.mat[sid] = []
        else:
            k, v = self.kv(sid)
            k = np.array(k[:, :n], copy=True)
            v = np.array(v[:, :n], copy=True)
            k.flags.writeable = False
            v.flags.writeable = False
            self.mat[sid] = [(k, v)]

    @staticmethod
    def check_path(parents: Sequence[int], accepted: Sequence[int]) -> None:
        """Raise InvalidError unless ``accepted`` is a chain from a root of
        the tree given by ``parents`` (parent index or -1 per node)."""
        n = len(parents)
        prev = -1
        for a in accepted:
            if not 0 <= a < n or parents[a] != prev:
                raise InvalidError("accepted nodes are not a chain from a root")
            prev = a

    def commit(self, sid: int, n_nodes: int, parents: Sequence[int], accepted: Sequence[int]):
        """Keep the accepted path of the draft tree that ends ``sid``.
        Returns the (slots, cow_ops) of the re-append."""
        self._check(sid)
        if n_nodes < 1 or n_nodes > self.lens[sid] or len(parents) != n_nodes:
            raise InvalidError("tree size does not fit the sequence")
        self.check_path(parents, accepted)
        c = self.lens[sid] - n_nodes
        k, v = self.kv(sid)
        pos = [c + a for a in accepted]
        kk = np.array(k[:, pos], copy=True)
        vv = np.array(v[:, pos], copy=True)
        snap, mat = self._snapshot(), list(self.mat[sid])
        self.truncate(sid, c)
        if not accepted:
            return [], []
        try:
            return self.append(sid, kk, vv)
        except OOMError:
            self._restore(snap)
            self.mat[sid] = mat
            raise

    def commit_batch(self, items):
        """Commit several draft trees of one verify step: ``items`` is a
        list of (sid, n_nodes, parents, accepted) for distinct sequences.
        Every request is truncated to its context first, then the kept paths
        are appended in list order; if an append runs out of blocks,
        everything is undone and ``OOMError`` is raised."""
        sids = [it[0] for it in items]
        if len(set(sids)) != len(sids):
            raise InvalidError("a sequence appears twice")
        gathered = []
        for sid, n_nodes, parents, accepted in items:
            self._check(sid)
            if n_nodes < 1 or n_nodes > self.lens[sid] or len(parents) != n_nodes:
                raise InvalidError("tree size does not fit the sequence")
            self.check_path(parents, accepted)
            c = self.lens[sid] - n_nodes
            k, v = self.kv(sid)
            pos = [c + a for a in accepted]
            gathered.append((c, np.array(k[:, pos], copy=True), np.array(v[:, pos], copy=True)))
        snap = self._snapshot()
        mats = {sid: list(self.mat[sid]) for sid in sids}
        for sid, (c, _, _) in zip(sids, gathered):
            self.truncate(sid, c)
        try:
            for sid, (_, kk, vv) in zip(sids, gathered):
                if kk.shape[1]:
                    self.append(sid, kk, vv)
        except OOMError:
            self._restore(snap)
            for sid in sids:
                self.mat[sid] = mats[sid]
            raise

    def free(self, sid: int) -> None:
        self._check(sid)
        for b in self.tables[sid]:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free_blocks.add(b)
        del self.tables[sid]
        del self.lens[sid]
        del self.mat[sid]

    # ----------------------------------------------------------- inspection
    def table(self, sid: int) -> List[int]:
        self._check(sid)
        return list(self.tables[sid])

    def length(self, sid: int) -> int:
        self._check(sid)
        return self.lens[sid]

    def refcount(self, b: int) -> int:
        return self.ref[b]

    def live(self) -> List[int]:
        return sorted(self.tables)

    def kv(self, sid: int, layer: Optional[int] = None):
        """The materialised (K, V) of ``sid`` as float32 arrays
        [L][len][Hkv][D], or [len][Hkv][D] for one ``layer``."""
        self._check(sid)
        chunks = self.mat[sid]
        if not chunks:
            raise InvalidError(f"sequence {sid} is empty")
        if layer is None:
            return (np.concatenate([c[0] for c in chunks], axis=1),
                    np.concatenate([c[1] for c in chunks], axis=1))
        return (np.concatenate([c[0][layer] for c in chunks], axis=0),
                np.concatenate([c[1][layer] for c in chunks], axis=0))


def run_trace(pool: OraclePool, ops, kv_for_op) -> Dict[int, int]:
    """Apply a workload's op trace to ``pool``. ``kv_for_op(i)`` gives the
    (K, V) float arrays of the append at op index ``i``. Returns the map from
    trace sid to pool sid (they are equal here)."""
    for i, op in enumerate(ops):
        if op.kind == "create":
            pool.create(op.sid)
        elif op.kind == "fork":
            pool.fork(op.parent, op.sid)
        elif op.kind == "append":
            k, v = kv_for_op(i)
            pool.append(op.sid, k, v)
        elif op.kind == "free":
            pool.free(op.sid)
        else:
            raise InvalidError(op.kind)
    return {s: s for s in pool.live()}
