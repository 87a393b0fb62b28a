"""Host side of libpkv through its C ABI (CPU only, no device calls).

Block tables, reference counts, free sets, slots and copy-on-write records
must equal the oracle's bit for bit on the same operation traces.
"""

from __future__ import annotations

import json
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from oracle.pool import OraclePool
from workloads import get

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def header_functions():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(pkv):
    from paged_kv_cache_amd import _lib
    declared = header_functions()
    assert len(declared) >= 20
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(pkv_\w+)", out))
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    assert set(_lib.declared_symbols()) == set(declared)
    for f in declared:
        getattr(_lib.lib, f)


def host_cache(pkv, nb, bs, order=None):
    return pkv.PagedKVCache(nb, bs, 1, 1, 1, 64, dtype="f32", device=None, alloc_order=order)


def zeros(n):
    return np.zeros((1, n, 1, 1), np.float32)


@pytest.mark.parametrize("name", ["tiny_a", "tiny_b"])
def test_tiny_tables_golden(pkv, name):
    gold = json.load(open(os.path.join(GOLDEN, "tiny_tables.json")))[name]
    w = get(name)
    c = host_cache(pkv, 16, w.shape.BS)
    h = {}
    cows = []
    first_slots = None
    for op in w.ops:
        if op.kind == "create":
            h[op.sid] = c.create()
        elif op.kind == "fork":
            h[op.sid] = c.fork(h[op.parent])
        elif op.kind == "append":
            slots, cw = c.plan(h[op.sid], op.n)
            cows += [list(x) for x in cw]
            if op.sid == 1:
                first_slots = slots
        elif op.kind == "free":
            c.free(h.pop(op.sid))
    for s, t in gold["tables"].items():
        assert c.table(h[int(s)]) == t
    for b, n in gold["refcounts"].items():
        assert c.refcount(int(b)) == n
    assert cows == gold["cow_ops"]
    assert first_slots == gold["first_branch_slots"]


def compare_state(c, pool: OraclePool, handles):
    assert sorted(handles) == pool.live()
    for sid, hd in handles.items():
        assert c.table(hd) == pool.table(sid)
        assert c.length(hd) == pool.length(sid)
    assert c.refcounts() == [pool.refcount(b) for b in range(pool.num_blocks)]
    st = c.stats()
    assert st["free_blocks"] == len(pool.free_blocks)
    assert st["live_seqs"] == len(pool.live())
    assert st["total_refs"] == sum(pool.ref)


@pytest.mark.parametrize("seed", range(16))
def test_random_traces_bit_exact(pkv, seed):
    rng = np.random.default_rng(100 + seed)
    nb = int(rng.integers(8, 48))
    bs = [1, 2, 4, 16][seed % 4]
    order = rng.permutation(nb).tolist() if seed % 2 else None
    c = host_cache(pkv, nb, bs, order)
    pool = OraclePool(nb, bs, alloc_order=order)
    handles = {}
    for _ in range(250):
        act = int(rng.integers(5)) if handles else 0
        if act == 0:
            sid = pool.create()
            handles[sid] = c.create()
        elif act == 1:
            p = list(handles)[rng.integers(len(handles))]
            sid = pool.fork(p)
            handles[sid] = c.fork(handles[p])
        elif act in (2, 3):
            sid = list(handles)[rng.integers(len(handles))]
            n = int(rng.integers(0, 3 * bs + 2))
            try:
                want = pool.append(sid, zeros(n), zeros(n))
            except oracle.OOMError:
                with pytest.raises(pkv.OOM):
                    c.plan(handles[sid], n)
            else:
                got = c.plan(handles[sid], n)
                assert got[0] == want[0]
                assert got[1] == [tuple(x) for x in want[1]]
        else:
            sid = list(handles)[rng.integers(len(handles))]
            pool.free(sid)
            c.free(handles.pop(sid))
        compare_state(c, pool, handles)
    for sid in list(handles):
        pool.free(sid)
        c.free(handles.pop(sid))
    st = c.stats()
    assert st["free_blocks"] == nb and st["total_refs"] == 0 and st["live_seqs"] == 0


@pytest.mark.parametrize("seed", range(8))
def test_random_traces_with_truncate_bit_exact(pkv, seed):
    """Forks, appends and truncations (as a draft-tree commit makes them)
    give the oracle's tables, counts and free list."""
    rng = np.random.default_rng(300 + seed)
    nb = int(rng.integers(12, 40))
    bs = [1, 2, 4, 16][seed % 4]
    order = rng.permutation(nb).tolist() if seed % 2 else None
    c = host_cache(pkv, nb, bs, order)
    pool = OraclePool(nb, bs, alloc_order=order)
    handles = {}
    for _ in range(200):
        act = int(rng.integers(5)) if handles else 0
        if act == 0:
            sid = pool.create()
            handles[sid] = c.create()
        elif act == 1:
            p = list(handles)[rng.integers(len(handles))]
            sid = pool.fork(p)
            handles[sid] = c.fork(handles[p])
        elif act == 2:
            sid = list(handles)[rng.integers(len(handles))]
            n = int(rng.integers(0, 3 * bs + 2))
            try:
                want = pool.append(sid, zeros(n), zeros(n))
            except oracle.OOMError:
                with pytest.raises(pkv.OOM):
                    c.plan(handles[sid], n)
            else:
                got = c.plan(handles[sid], n)
                assert got[0] == want[0]
                assert got[1] == [tuple(x) for x in want[1]]
        elif act == 3:
            sid = list(handles)[rng.integers(len(handles))]
            n = int(rng.integers(0, pool.length(sid) + 1))
            pool.truncate(sid, n)
            c.truncate(handles[sid], n)
        else:
            sid = list(handles)[rng.integers(len(handles))]
            pool.free(sid)
            c.free(handles.pop(sid))
        compare_state(c, pool, handles)


@pytest.mark.parametrize("seed", range(6))
def test_long_tables_across_chunks_bit_exact(pkv, seed):
    """Tables of hundreds of blocks (several 64-id chunks of the persistent
    table): forks of forks, appends and truncations that cross chunk
    boundaries, copy-on-write of shared tails, frees; tables and counts
    equal the oracle's after every step."""
    rng = np.random.default_rng(900 + seed)
    bs = [1, 2][seed % 2]
    nb = 1200
    order = rng.permutation(nb).tolist() if seed % 3 == 0 else None
    c = host_cache(pkv, nb, bs, order)
    pool = OraclePool(nb, bs, alloc_order=order)
    root = pool.create()
    handles = {root: c.create()}
    n = int(rng.integers(150, 300)) * bs + int(rng.integers(bs))
    pool.append(root, zeros(n), zeros(n))
    c.plan(handles[root], n)
    for _ in range(120):
        act = int(rng.integers(5))
        sid = list(handles)[rng.integers(len(handles))]
        if act == 0 and len(handles) < 12:
            k = pool.fork(sid)
            handles[k] = c.fork(handles[sid])
        elif act in (1, 2):
            m = int(rng.integers(0, 70 * bs))
            try:
                want = pool.append(sid, zeros(m), zeros(m))
            except oracle.OOMError:
                with pytest.raises(pkv.OOM):
                    c.plan(handles[sid], m)
            else:
                got = c.plan(handles[sid], m)
                assert got[0] == want[0] and got[1] == [tuple(x) for x in want[1]]
        elif act == 3:
            m = int(rng.integers(0, pool.length(sid) + 1))
            pool.truncate(sid, m)
            c.truncate(handles[sid], m)
        elif len(handles) > 1:
            pool.free(sid)
            c.free(handles.pop(sid))
        compare_state(c, pool, handles)


def test_fork_cost_does_not_grow_with_the_table(pkv):
    """A fork shares the parent's table: forking (and freeing) a 16,384-block
    sequence copies no block id, however long the table, where a table copy
    would write 16,384 of them. The first append to a fork copies only the
    parts it changes: the list of chunk references (one per 64 ids) and the
    last chunk. Counted by the pool (table_ids_copied), not timed."""
    c = host_cache(pkv, 20000, 1)
    small, big = c.create(), c.create()
    c.plan(small, 16)
    c.plan(big, 16384)
    for seq, n in ((small, 16), (big, 16384)):
        before = c.stats()["table_ids_copied"]
        kids = [c.fork(seq) for _ in range(100)]
        for k in kids:
            assert c.table(k) == c.table(seq)
        assert all(c.refcount(b) == 101 for b in c.table(seq)[:5])
        c.free_many(kids)
        assert c.stats()["table_ids_copied"] == before, n
    # the first append to a fork of the 16,384-block table (block size 1, so
    # the tail is full and only the list is copied): 256 chunk references
    k = c.fork(big)
    before = c.stats()["table_ids_copied"]
    c.plan(k, 1)
    assert c.stats()["table_ids_copied"] - before == 16384 // 64
    assert c.table(k)[:-1] == c.table(big) and c.refcount(c.table(big)[0]) == 2


def test_truncate_rejects_bad_lengths(pkv):
    from paged_kv_cache_amd import binding
    c = host_cache(pkv, 8, 4)
    s = c.create()
    c.plan(s, 6)
    for n in (-1, 7):
        with pytest.raises(pkv.PkvError) as e:
            c.truncate(s, n)
        assert e.value.code == pkv.PKV_E_INVALID
    assert c.length(s) == 6 and c.table(s) == [0, 1]
    c.truncate(s, 6)
    assert c.table(s) == [0, 1]
    c.truncate(s, 0)
    assert c.table(s) == [] and c.stats()["free_blocks"] == 8
    with pytest.raises(pkv.PkvError):      # device call without arenas
        binding.pkv_tree_commit(c.handle, s, [-1], [0], None)


@pytest.mark.parametrize("seed", range(12))
def test_prompt_cache_traces_bit_exact(pkv, seed):
    """Random traces that mix the prompt cache (insert, match, clear, a
    capacity) with forks, appends, truncations and frees in a pool small
    enough to force evictions: tables, counts, free lists, cache sizes and
    match results equal the oracle's."""
    rng = np.random.default_rng(700 + seed)
    nb = int(rng.integers(16, 48))
    bs = [1, 2, 4, 16][seed % 4]
    order = rng.permutation(nb).tolist() if seed % 2 else None
    cap = [nb, 3, 8, 0][seed % 4] if seed >= 4 else nb
    c = host_cache(pkv, nb, bs, order)
    c.set_option("prefix_cache_blocks", cap)
    pool = OraclePool(nb, bs, alloc_order=order)
    pool.cache_capacity = cap
    handles, toks = {}, {}
    vocab = 3 if bs <= 2 else 2

    def new_ids(n):
        return [int(t) for t in rng.integers(0, vocab, size=n)]

    for _ in range(300):
        act = int(rng.integers(8)) if handles else 0
        if act == 0:
            q = new_ids(int(rng.integers(0, 3 * bs + 2)))
            if handles and rng.integers(2):      # resume a known conversation
                src = toks[list(handles)[rng.integers(len(handles))]]
                q = src[:int(rng.integers(0, len(src) + 1))] + q
            sid, m = pool.cache_match(q)
            hd, m2 = c.cache_match(q)
            assert m2 == m
            handles[sid], toks[sid] = hd, q[:m]
        elif act == 1:
            p = list(handles)[rng.integers(len(handles))]
            sid = pool.fork(p)
            handles[sid], toks[sid] = c.fork(handles[p]), list(toks[p])
        elif act in (2, 3):
            sid = list(handles)[rng.integers(len(handles))]
            n = int(rng.integers(0, 2 * bs + 2))
            try:
                want = pool.append(sid, zeros(n), zeros(n))
            except oracle.OOMError:
                with pytest.raises(pkv.OOM):
                    c.plan(handles[sid], n)
            else:
                got = c.plan(handles[sid], n)
                assert got[0] == want[0]
                assert got[1] == [tuple(x) for x in want[1]]
                toks[sid] += new_ids(n)
        elif act == 4:
            sid = list(handles)[rng.integers(len(handles))]
            n = int(rng.integers(0, len(toks[sid]) + 1))
            assert pool.cache_insert(sid, toks[sid][:n]) == c.cache_insert(handles[sid], toks[sid][:n])
        elif act == 5:
            sid = list(handles)[rng.integers(len(handles))]
            n = int(rng.integers(0, pool.length(sid) + 1))
            pool.truncate(sid, n)
            c.truncate(handles[sid], n)
            toks[sid] = toks[sid][:n]
        elif act == 6:
            sid = list(handles)[rng.integers(len(handles))]
            pool.free(sid)
            c.free(handles.pop(sid))
            del toks[sid]
        elif rng.integers(4) == 0:
            pool.cache_clear()
            c.cache_clear()
        compare_state(c, pool, handles)
        assert c.cache_info() == (len(pool.entries), pool.evictable())
    for sid in list(handles):
        pool.free(sid)
        c.free(handles.pop(sid))
    c.cache_clear()
    st = c.stats()
    assert st["free_blocks"] == nb and st["total_refs"] == 0


def test_prompt_cache_eviction_order_matches_hand_derivation(pkv):
    """The oracle's hand-derived case: evictions free blocks 1, 2, then 0."""
    c = host_cache(pkv, 6, 2)
    a, b = c.create(), c.create()
    c.plan(a, 4)
    c.plan(b, 2)
    assert c.cache_insert(a, [1, 2, 3, 4]) == 2 and c.cache_insert(b, [5, 6]) == 1
    m, n = c.cache_match([1, 2, 9])
    assert n == 2 and c.table(m) == [0]
    for s in (m, a, b):
        c.free(s)
    assert c.cache_info() == (3, 3)
    d = c.create()
    c.plan(d, 6)
    assert c.table(d) == [3, 4, 5]
    for want in (1, 2, 0):
        c.plan(d, 2)
        assert c.table(d)[-1] == want
    assert c.cache_info() == (0, 0)
    with pytest.raises(pkv.OOM):
        c.plan(d, 1)
    with pytest.raises(pkv.PkvError):
        c.cache_insert(d, list(range(13)))      # more ids than tokens
    with pytest.raises(pkv.PkvError):
        c.set_option("prefix_cache_blocks", 7)  # above num_blocks


@pytest.mark.parametrize("name", ["beam", "mcts", "agent", "verify", "beam_cow"])
def test_full_size_tables_bit_exact(pkv, name):
    w = get(name)
    nb = w.num_blocks_bound()
    c = host_cache(pkv, nb, w.shape.BS)
    pool = OraclePool(nb, w.shape.BS)
    handles = {}
    for op in w.ops:
        if op.kind == "create":
            pool.create(op.sid)
            handles[op.sid] = c.create()
        elif op.kind == "fork":
            pool.fork(op.parent, op.sid)
            handles[op.sid] = c.fork(handles[op.parent])
        elif op.kind == "append":
            want = pool.append(op.sid, zeros(op.n), zeros(op.n))
            got = c.plan(handles[op.sid], op.n)
            assert got[0] == want[0] and got[1] == [tuple(x) for x in want[1]]
        else:
            pool.free(op.sid)
            c.free(handles.pop(op.sid))
    compare_state(c, pool, handles)


def test_batch_append_equals_sequential(pkv):
    """Batch planning follows sequence order: when two batch members share a
    partly filled tail, the first copies it and the second, now its only
    holder, writes in place."""
    for order in (None, list(np.random.default_rng(5).permutation(40))):
        a = host_cache(pkv, 40, 4, order)
        b = host_cache(pkv, 40, 4, order)
        ra, rb = a.create(), b.create()
        a.plan(ra, 6)
        b.plan(rb, 6)
        ka = [a.fork(ra) for _ in range(3)]
        kb = [b.fork(rb) for _ in range(3)]
        a.free(ra)
        b.free(rb)
        counts = [3, 0, 5]
        from paged_kv_cache_amd import binding
        # batch planning without device work: the arenas are absent, so use
        # the planner through sequential plan() calls on one pool and the
        # batch call's table outcome on the other
        for k, n in zip(ka, counts):
            a.plan(k, n)
        with pytest.raises(pkv.PkvError):
            binding.pkv_append_kv_batch(b.handle, kb, counts, None, None)   # no arenas: rejected
        for k, n in zip(kb, counts):
            b.plan(k, n)
        for x, y in zip(ka, kb):
            assert a.table(x) == b.table(y)


def visible_stats(c):
    """The pool's state as callers see it (without the work counter
    table_ids_copied, which a refused call may advance: it copies private
    table parts before it counts blocks, invisibly)."""
    st = dict(c.stats())
    st.pop("table_ids_copied")
    return st


def test_oom_is_atomic_and_reported(pkv):
    c = host_cache(pkv, 3, 4)
    s = c.create()
    c.plan(s, 6)
    k = c.fork(s)
    before = (c.table(s), c.table(k), [c.refcount(b) for b in range(3)], visible_stats(c))
    with pytest.raises(pkv.OOM):
        c.plan(k, 4)            # needs a copy + a fresh block, one is free
    assert (c.table(s), c.table(k), [c.refcount(b) for b in range(3)], visible_stats(c)) == before
    c.plan(k, 2)
    assert c.table(k) == [0, 2] and c.refcount(1) == 1


def test_invalid_handles_and_arguments(pkv):
    from paged_kv_cache_amd import binding
    c = host_cache(pkv, 8, 4)
    s = c.create()
    c.plan(s, 3)
    c.free(s)
    for fn in (lambda: c.free(s), lambda: c.fork(s), lambda: c.plan(s, 1), lambda: c.table(s)):
        with pytest.raises(pkv.PkvError) as e:
            fn()
        assert e.value.code == pkv.PKV_E_INVALID
    with pytest.raises(pkv.PkvError):
        binding.pkv_block_release(c.handle, 5)     # free block
    with pytest.raises(pkv.PkvError):
        binding.pkv_block_refcount(c.handle, 8)    # out of range
    with pytest.raises(pkv.PkvError):
        binding.pkv_pool_set_option(c.handle, "no_such_option", 1)
    # the streaming-read measuring aid checks its arguments before any device work
    from paged_kv_cache_amd import _lib
    for src, nbytes, nt in ((4096, 17, 1), (4096, 0, 1), (4104, 4096, 1), (4096, 4096, 2), (None, 4096, 1)):
        assert _lib.lib.pkv_stream_read(src, nbytes, nt, 4096, None) == pkv.PKV_E_INVALID
    for v in (0, 1, 2):
        binding.pkv_pool_set_option(c.handle, "wide_spec", v)
    for v in (-1, 3):
        with pytest.raises(pkv.PkvError):
            binding.pkv_pool_set_option(c.handle, "wide_spec", v)
    t = c.create()
    with pytest.raises(pkv.PkvError):
        c.plan(t, -1)
    with pytest.raises(pkv.PkvError):      # device call without arenas
        binding.pkv_cow_copy(c.handle, [(0, 1, 1)])
    with pytest.raises(pkv.PkvError):      # bad desc
        binding.pkv_pool_create(4, 16, 1, 3, 4, 64, 0)
    with pytest.raises(pkv.PkvError):      # not a permutation
        binding.pkv_pool_create(4, 16, 1, 1, 1, 64, 0, alloc_order=[0, 1, 1, 2])
    b = binding.pkv_block_alloc(c.handle)
    assert c.refcount(b) == 1
    binding.pkv_block_release(c.handle, b)
    assert c.refcount(b) == 0


def test_fork_leaves_parent_unchanged(pkv):
    c = host_cache(pkv, 64, 4)
    p = c.create()
    c.plan(p, 10)
    t0 = c.table(p)
    kids = [c.fork(p) for _ in range(5)]
    assert c.table(p) == t0 and c.length(p) == 10
    for k in kids:
        c.plan(k, 3)
        assert c.table(p) == t0 and c.length(p) == 10
    assert [c.refcount(b) for b in t0] == [6, 6, 1]   # the shared tail was copied by all 5


def distinct_tokens(c, handles):
    seen = {}
    for h in handles:
        n = c.length(h)
        for j, b in enumerate(c.table(h)):
            seen[b] = min(c.BS, n - j * c.BS)
    return sum(seen.values())


@pytest.mark.parametrize("name,segments", [("tiny_a", 5), ("tiny_b", 5), ("beam", 9), ("mcts", 127),
                                           ("agent", 5)])
def test_plan_segments_closed_form(pkv, name, segments):
    """Segments: the shared root plus one per private tail (star trees);
    the root plus one per edge of the binary tree (126 edges + 1)."""
    w = get(name)
    c = pkv.PagedKVCache(w.num_blocks_bound(), w.shape.BS, w.shape.L, w.shape.Hkv, w.shape.Hq,
                         w.shape.D, dtype=w.shape.dtype, device=None)
    h = {}
    for op in w.ops:
        if op.kind == "create":
            h[op.sid] = c.create()
        elif op.kind == "fork":
            h[op.sid] = c.fork(h[op.parent])
        elif op.kind == "append":
            c.plan(h[op.sid], op.n)
        else:
            c.free(h.pop(op.sid))
    seqs = [h[s] for s in w.query_sids]
    c.set_option("fold_tokens", 0)
    info = c.plan_info(seqs)
    assert info["n_segments"] == segments
    assert info["unique_tokens"] == distinct_tokens(c, seqs)
    assert info["n_chunks"] >= segments
    assert info["workspace_bytes"] > 0


def test_plan_bytes_and_the_inline_limit(pkv):
    """The plan's arrays are packed at 16-byte alignment: the beam step's plan
    (9 items, 256 block ids, 16 holders, the combine lists) and the MCTS plan
    (17 items, 576 block ids and their block words) fit the 12,288 bytes a
    launch carries in its arguments, so neither needs a plan upload; the
    agent's (190 items, 1,440 block ids) does not and is staged. The
    workspace holds the plan, then the partial states."""
    G = 4
    for name, inline in (("beam", True), ("mcts", True), ("agent", False)):
        w = get(name)
        c, seqs = build_host_tree(pkv, w)
        info = c.plan_info(seqs)
        pb = info["plan_bytes"]
        assert pb % 16 == 0 and pb >= info["n_items"] * 48 + 4 * (len(seqs) + 1), (name, pb)
        assert (pb <= 12288) == inline, (name, pb)
        part = info["partial_rows"] * w.shape.L * w.shape.Hkv * (w.shape.D + 2) * 4
        assert info["workspace_bytes"] >= pb + part, name
    w = get("beam")
    c, seqs = build_host_tree(pkv, w)
    info = c.plan_info(seqs)
    # 9 items (the root's 32 rows, then 8 private tails of 4 rows) x 48 B,
    # 128 + 8 x 16 block ids, 8 + 8 holders, 9 + 16 list entries
    assert info["n_items"] == 9
    assert info["plan_bytes"] == 432 + 1024 + 64 + 48 + 64


def test_plan_folds_short_edges_per_leaf(pkv):
    """With fold_tokens above the MCTS edge length (32 tokens), every leaf
    reads its 6 edges (the 5 shared ones and its own) as one item: chunks =
    the root's + one per leaf, and the partial rows per plane drop from one
    per (edge, row) to one per leaf row; segments and unique tokens describe
    the tree as before."""
    w = get("mcts")
    c, seqs = build_host_tree(pkv, w)
    G = w.shape.Hq // w.shape.Hkv
    c.set_option("tree", 0)          # (the narrow / wide items' plan)
    c.set_option("group_rows", 0)    # (one item per leaf)
    c.set_option("fold_tokens", 0)
    plain = c.plan_info(seqs)
    c.set_option("fold_tokens", 64)
    folded = c.plan_info(seqs)
    assert plain["n_segments"] == folded["n_segments"] == 127
    assert plain["unique_tokens"] == folded["unique_tokens"]
    root_chunks = plain["n_chunks"] - 126
    assert folded["n_chunks"] == root_chunks + 64
    assert plain["partial_rows"] == root_chunks * 64 * G + 6 * 64 * G
    assert folded["partial_rows"] == root_chunks * 64 * G + 64 * G
    # every token slot once, then the root once and each leaf's 6 edges
    assert plain["read_tokens"] == plain["unique_tokens"] == 4096 + 126 * 32
    assert folded["read_tokens"] == 4096 + 64 * 6 * 32
    assert plain["grouped_items"] == folded["grouped_items"] == 0
    c.set_option("fold_tokens", 16)                    # shorter than the edges: no folding
    assert c.plan_info(seqs) == plain


def test_plan_groups_sibling_leaves(pkv):
    """With grouping (option group_rows, 16 by default), the four leaves under
    each depth-4 node of the MCTS tree (4 x G = 16 rows) share one item that
    reads their path's 10 distinct edges once (4 shared, 2 at depth 5, 4 at
    depth 6) instead of 4 x 6: 16 items, 16 chunks and 320 tokens each, and
    one partial row per leaf row as with one item per leaf. With 8 rows,
    pairs of sibling leaves (7 edges for 2 x 6); with 4 rows (one leaf), no
    group. The order of the batch does not matter: siblings are found by
    their blocks."""
    w = get("mcts")
    c, seqs = build_host_tree(pkv, w)
    G = w.shape.Hq // w.shape.Hkv
    assert G == 4
    c.set_option("tree", 0)
    c.set_option("group_rows", 0)
    single = c.plan_info(seqs)
    c.set_option("group_rows", 16)
    quads = c.plan_info(seqs)
    root_chunks = single["n_chunks"] - 64
    assert quads["grouped_items"] == 16
    assert quads["n_chunks"] == root_chunks + 16
    assert quads["partial_rows"] == single["partial_rows"]
    assert quads["read_tokens"] == 4096 + 16 * 10 * 32
    assert quads["unique_tokens"] == single["unique_tokens"]
    c.set_option("group_rows", 8)
    pairs = c.plan_info(seqs)
    assert pairs["grouped_items"] == 32
    assert pairs["read_tokens"] == 4096 + 32 * 7 * 32
    c.set_option("group_rows", 4)
    assert c.plan_info(seqs) == single
    c.set_option("group_rows", 16)
    shuffled = [seqs[i] for i in np.random.default_rng(3).permutation(len(seqs))]
    again = c.plan_info(shuffled)
    assert again["grouped_items"] == 16 and again["read_tokens"] == quads["read_tokens"]
    c.set_option("rows_per_item", 8)                   # groups fit a narrow item
    assert c.plan_info(seqs)["read_tokens"] == 4096 + 32 * 7 * 32


def test_plan_groups_only_what_shares(pkv):
    """Branches whose folded paths share less than a quarter of their blocks
    stay one item each: 8 forks of a 40-token root (its 2 full blocks shared,
    32 tokens, folded) that each append 400 tokens read 2 + 26 blocks each
    (the root's partly filled block copied, then 25 more), a group of four
    2 + 104 of 112 blocks. Forks of a 60-token root (3 shared blocks) that
    append 20 tokens (2 blocks of their own) form groups: 3 + 8 of 20."""
    c = pkv.PagedKVCache(512, 16, 1, 2, 8, 64, dtype="bf16", device=None)
    root = c.create()
    c.plan(root, 40)
    kids = [c.fork(root) for _ in range(8)]
    for k in kids:
        c.plan(k, 400)
    info = c.plan_info(kids)
    assert info["grouped_items"] == 0
    assert info["read_tokens"] == 8 * (48 + 400)
    c2 = pkv.PagedKVCache(512, 16, 1, 2, 8, 64, dtype="bf16", device=None)
    r2 = c2.create()
    c2.plan(r2, 60)
    kids2 = [c2.fork(r2) for _ in range(8)]
    for k in kids2:
        c2.plan(k, 20)
    info2 = c2.plan_info(kids2)
    assert info2["grouped_items"] == 2


def test_plan_tree_for_mcts(pkv):
    """The MCTS batch (64 leaves x G = 4 = 256 rows, 256 planes) takes the
    tree plan when asked (option tree 1): one item, the root cut into 8
    pieces of 512 tokens and the 126 edges whole (134 chunks), each token
    slot read once (unique tokens as for the other plan), no partial states.
    Off by default (tree 0); with tree 1 not taken when the planes do not
    fill the chip (a one-layer call) unless forced (tree 2), nor when the
    rows do not fit one workgroup."""
    w = get("mcts")
    c, seqs = build_host_tree(pkv, w)
    items = c.plan_info(seqs)
    assert items["partial_rows"] > 0
    c.set_option("tree", 1)
    tree = c.plan_info(seqs)
    assert tree["n_chunks"] == 4096 // 512 + 126
    assert tree["n_items"] == 0 and tree["partial_rows"] == 0
    assert tree["unique_tokens"] == distinct_tokens(c, seqs) == 4096 + 126 * 32
    assert items["unique_tokens"] == tree["unique_tokens"]
    assert tree["workspace_bytes"] == (tree["plan_bytes"] + 255) // 256 * 256   # the plan alone
    c.set_option("tree_piece_tokens", 1024)
    assert c.plan_info(seqs)["n_chunks"] == 4 + 126
    c.set_option("tree_piece_tokens", 512)
    c.set_option("tree", 0)
    assert c.plan_info(seqs)["partial_rows"] > 0
    c.set_option("tree", 1)
    one_layer = c.plan_info(seqs, n_layers=1)         # 8 planes: the root is split for parallelism
    assert one_layer["partial_rows"] > 0
    c.set_option("tree", 2)
    assert c.plan_info(seqs, n_layers=1)["partial_rows"] == 0
    # 65 branches x G = 4 = 260 rows: more than one workgroup holds
    more = c.fork_many(seqs[:1])
    assert c.plan_info(seqs + more)["partial_rows"] > 0


def build_host_tree(pkv, w):
    c = pkv.PagedKVCache(w.num_blocks_bound(), w.shape.BS, w.shape.L, w.shape.Hkv, w.shape.Hq,
                         w.shape.D, dtype=w.shape.dtype, device=None)
    h = {}
    for op in w.ops:
        if op.kind == "create":
            h[op.sid] = c.create()
        elif op.kind == "fork":
            h[op.sid] = c.fork(h[op.parent])
        elif op.kind == "append":
            c.plan(h[op.sid], op.n)
        else:
            c.free(h.pop(op.sid))
    return c, [h[s] for s in w.query_sids]


@pytest.mark.parametrize("name,chunks", [("agent", 1 + 4 * 2), ("beam", 9)])
def test_plan_caps_chunks_at_512_blocks(pkv, name, chunks):
    """However long the requested chunks, none spans more than 512 blocks
    (the matrix-core kernels stage a chunk's block ids in LDS): agent's
    416-block prefix stays whole and each 1024-block tail splits in two."""
    w = get(name)
    c, seqs = build_host_tree(pkv, w)
    c.set_option("chunk_tokens", 1 << 20)
    assert c.plan_info(seqs)["n_chunks"] == chunks


def test_fork_many_and_free_many(pkv):
    c = host_cache(pkv, 32, 4)
    p = c.create()
    c.plan(p, 6)
    kids = c.fork_many([p, p, p])
    assert [c.table(k) for k in kids] == [c.table(p)] * 3
    assert [c.refcount(b) for b in c.table(p)] == [4, 4]
    before = c.stats()
    stale = c.create()
    c.free(stale)
    with pytest.raises(pkv.PkvError):
        c.fork_many([p, stale])          # all or nothing
    assert c.stats() == before
    with pytest.raises(pkv.PkvError):
        c.free_many([kids[0], kids[0]])  # listed twice
    assert c.stats() == before
    c.free_many(kids)
    assert [c.refcount(b) for b in c.table(p)] == [1, 1]
    assert c.stats()["live_seqs"] == 1


@pytest.mark.parametrize("name,min_chunk,per_row", [("agent", 768, 32), ("beam", 1024, 64), ("mcts", 1024, 64)])
def test_chunk_defaults_follow_head_size(pkv, name, min_chunk, per_row):
    """min_chunk_tokens / tokens_per_row 0 (the default) resolve by head
    size: 768 and 32 above 128 dims (the agent tree, D = 256), 1024 and 64
    up to 128 (beam, MCTS); set explicitly, the plan is the same."""
    w = get(name)
    c, seqs = build_host_tree(pkv, w)
    auto = c.plan_info(seqs)
    c.set_option("min_chunk_tokens", min_chunk)
    c.set_option("tokens_per_row", per_row)
    assert c.plan_info(seqs) == auto
    c.set_option("min_chunk_tokens", 0)
    c.set_option("tokens_per_row", 0)
    assert c.plan_info(seqs) == auto


def test_plan_truncated_fork_beside_its_sibling(pkv):
    """After a truncate two holders can see different valid counts in one
    block (A holds 40 tokens, its fork B was cut to 36: block 2 holds 8 of
    A's tokens and 4 of B's). Decode plans such a batch: the shared blocks
    0-1 form one segment read once for both; block 2 is read by each holder
    on its own, up to its own length."""
    c = host_cache(pkv, 16, 16)
    a = c.create()
    c.plan(a, 40)
    b = c.fork(a)
    c.truncate(b, 36)
    assert c.table(b) == c.table(a) == [0, 1, 2]
    c.set_option("fold_tokens", 0)
    info = c.plan_info([a, b])
    # segments: blocks 0-1 for {A, B}; block 2 for {A} (8 tokens) and for {B} (4)
    assert info["n_segments"] == 3
    assert info["unique_tokens"] == 32 + 8 + 4
    info2 = c.plan_info([b, a])
    assert info2["n_segments"] == 3 and info2["unique_tokens"] == 44
    # a third holder agreeing with A: still one read per holder of block 2
    d = c.fork(a)
    assert c.plan_info([a, b, d])["unique_tokens"] == 32 + 8 + 4 + 8
    # A grows past block 2 (copying it on write, B keeps the original)
    c.free(d)
    c.plan(a, 20)
    assert c.table(a)[:2] == [0, 1] and c.table(a)[2] != 2 and c.table(b) == [0, 1, 2]
    assert c.plan_info([a, b])["n_segments"] == 3


def test_null_arrays_after_a_cached_plan(pkv):
    """A call with a null sequence (or parent) array is refused with
    PKV_E_INVALID, also right after a successful call of the same size whose
    plan is cached (the cache comparison must not read through the null)."""
    import ctypes
    from paged_kv_cache_amd import _lib
    c = host_cache(pkv, 16, 16)
    a = c.create()
    c.plan(a, 20)
    b = c.fork(a)
    c.plan_info([a, b])
    size = ctypes.c_size_t(0)
    assert _lib.lib.pkv_decode_workspace_size(c.handle, None, 2, 1, ctypes.byref(size)) == \
        pkv.PKV_E_INVALID
    info = _lib.PkvPlanInfo()
    assert _lib.lib.pkv_decode_plan_info(c.handle, None, 2, 1, ctypes.byref(info)) == \
        pkv.PKV_E_INVALID
    assert _lib.lib.pkv_decode_attn(c.handle, None, 2, 0, 1, None, None, ctypes.c_float(1.0),
                                    None, 0, None) == pkv.PKV_E_INVALID
    assert _lib.lib.pkv_tree_verify_attn(c.handle, None, 1, None, 4, 0, None, None,
                                         ctypes.c_float(1.0), None, 0, None) == pkv.PKV_E_INVALID
