"""Committing a verified draft-tree path on the device, against the oracle.

Tables, reference counts and the K/V bytes every live sequence reads are
bit-exact; attention over the committed sequences meets the decode bar
(max |error| <= 2e-3, relative L2 <= 1e-2 against float64).
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import configs, generate, scaled  # noqa: E402
from workloads.configs import replace_shape  # noqa: E402
from workloads.gen import draw, verify_parents  # noqa: E402

from gpu_helpers import (arena_bits, build_library, build_oracle, errors, gather,  # noqa: E402
                         raw_bits, to_device)

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-3
REL_L2 = 1e-2


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def root_path(parents, leaf):
    path = []
    while leaf != -1:
        path.append(int(leaf))
        leaf = int(parents[leaf])
    return path[::-1]


def same_state(c, h, pool, what):
    """Tables, counts and every live sequence's K/V bits equal the oracle's."""
    torch.cuda.synchronize()
    kb, vb = arena_bits(c.k_arena), arena_bits(c.v_arena)
    assert sorted(h) == pool.live(), what
    for sid, hd in h.items():
        assert c.table(hd) == pool.table(sid), (what, sid)
        assert c.length(hd) == pool.length(sid), (what, sid)
        if pool.length(sid):
            K, V = gather(c, kb, vb, hd)
            Ko, Vo = pool.kv(sid)
            assert np.array_equal(K, raw_bits(Ko, c.dtype)), (what, sid)
            assert np.array_equal(V, raw_bits(Vo, c.dtype)), (what, sid)
    for b in range(pool.num_blocks):
        assert c.refcount(b) == pool.refcount(b), (what, b)
    assert c.stats()["free_blocks"] == len(pool.free_blocks), what


def check_close(got, want, what):
    ma, rl = errors(got, want)
    note(f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e}")
    assert np.all(np.isfinite(got)), what
    assert ma <= MAX_ABS and rl <= REL_L2, (what, ma, rl)


AG = configs.AGENT
B16 = configs.BEAM

COMMIT_CASES = [
    scaled("verify", "commit_s", shape=replace_shape(AG, Hq=12, Hkv=2), n_req=3, ctx_len=200,
           n_nodes=13, max_depth=4),
    scaled("verify", "commit_d128_bs16", shape=replace_shape(B16, L=2, Hq=8, Hkv=2), n_req=3,
           ctx_len=77, n_nodes=48, max_depth=8),
    scaled("verify", "commit_64nodes_bs64", shape=replace_shape(AG, Hq=4, Hkv=1, D=64, BS=64),
           n_req=2, ctx_len=64, n_nodes=64, max_depth=64),
    scaled("verify", "commit_noctx", shape=replace_shape(AG, Hq=6, Hkv=3, D=128), n_req=2, ctx_len=0,
           n_nodes=20, max_depth=5),
]


@pytest.mark.parametrize("w", COMMIT_CASES, ids=lambda w: w.name)
def test_commit_matches_oracle(pkv, w):
    """One request keeps a random root path, one keeps nothing, one keeps its
    deepest path; a fork of the first request, taken before the commit,
    shares its context tail and must still read the whole tree afterwards.
    Decode over the committed requests then agrees with the oracle."""
    note(f"commit {w.name}")
    inp = generate(w)
    c, h = build_library(pkv, w, inp)
    pool = build_oracle(w, inp)
    same_state(c, h, pool, f"{w.name} before the commit")
    reqs = list(w.query_sids)
    fsid = pool.fork(reqs[0])
    h[fsid] = c.fork(h[reqs[0]])
    rng = np.random.default_rng(5)
    N = w.n_nodes
    for r, sid in enumerate(reqs):
        par = [int(x) for x in inp.parents[r]]
        if r % 3 == 1:
            path = []
        elif r % 3 == 2:
            depth = [len(root_path(par, j)) for j in range(N)]
            path = root_path(par, int(np.argmax(depth)))
        else:
            path = root_path(par, int(rng.integers(N)))
        note(f"  request {r}: keep {len(path)} of {N} nodes")
        pool.commit(sid, N, par, path)
        c.commit(h[sid], par, path)
        same_state(c, h, pool, f"{w.name} after request {r}")
    sh = w.shape
    live = [s for s in reqs + [fsid] if pool.length(s) > 0]
    q = draw(np.random.default_rng(9), (sh.L, len(live), sh.Hq, sh.D), "bf16")
    got = c.decode([h[s] for s in live], to_device(q), scale=w.softmax_scale)
    torch.cuda.synchronize()
    want = oracle.decode(pool, live, q.f32(), w.softmax_scale)
    check_close(got.cpu().numpy(), want, f"decode after commit {w.name}")
    c.close()


@pytest.mark.parametrize("seed,bs,D", [(0, 16, 128), (1, 32, 128), (2, 64, 64), (3, 16, 256)])
def test_speculative_steps_match_oracle(pkv, seed, bs, D):
    """Repeated draft / verify / commit steps: each step appends a random
    draft tree to every request, verifies it (tree attention against the
    oracle), keeps a random root path, and sometimes forks a request."""
    note(f"speculative steps seed={seed} bs={bs} D={D}")
    L, Hkv, Hq = 2, 2, 8
    rng = np.random.default_rng(2000 + seed)
    nb = 160
    c = pkv.PagedKVCache(nb, bs, L, Hkv, Hq, D, dtype="bf16", device="cuda")
    pool = oracle.OraclePool(nb, bs)
    h = {}
    for _ in range(2):
        sid = pool.create()
        h[sid] = c.create()
        n = int(rng.integers(1, 3 * bs))
        k = draw(rng, (L, n, Hkv, D), "bf16")
        v = draw(rng, (L, n, Hkv, D), "bf16")
        pool.append(sid, k.f32(), v.f32())
        c.append([h[sid]], [n], to_device(k), to_device(v))
    scale = D ** -0.5
    for step in range(6):
        reqs = sorted(h)
        N = int(rng.integers(1, 65))
        parents = np.stack([verify_parents(seed * 100 + step, r, N, 6) for r in range(len(reqs))])
        k = draw(rng, (L, N * len(reqs), Hkv, D), "bf16")
        v = draw(rng, (L, N * len(reqs), Hkv, D), "bf16")
        for i, sid in enumerate(reqs):
            pool.append(sid, k.f32()[:, i * N:(i + 1) * N], v.f32()[:, i * N:(i + 1) * N])
        c.append([h[s] for s in reqs], [N] * len(reqs), to_device(k), to_device(v))
        q = draw(rng, (len(reqs), N, Hq, D), "bf16")
        got = c.verify([h[s] for s in reqs], parents, to_device(q), scale=scale)
        torch.cuda.synchronize()
        want = oracle.verify(pool, reqs, parents, q.f32(), scale)
        check_close(got.cpu().numpy(), want, f"step {step} verify ({len(reqs)} x {N} nodes)")
        for i, sid in enumerate(reqs):
            par = [int(x) for x in parents[i]]
            path = root_path(par, int(rng.integers(N)))
            pool.commit(sid, N, par, path)
            c.commit(h[sid], par, path)
        if step % 2 == 0 and len(h) < 5:
            p = reqs[int(rng.integers(len(reqs)))]
            sid = pool.fork(p)
            h[sid] = c.fork(h[p])
        same_state(c, h, pool, f"step {step}")
    c.close()


def test_commit_errors_change_nothing(pkv):
    """A path that is not a chain from a root, a tree longer than the
    sequence, a too-small workspace, and a commit that runs out of blocks
    are all rejected with the tables and the arena unchanged."""
    from paged_kv_cache_amd import binding
    L, Hkv, Hq, D, bs = 1, 1, 2, 64, 16
    c = pkv.PagedKVCache(2, bs, L, Hkv, Hq, D, dtype="bf16", device="cuda")
    pool = oracle.OraclePool(2, bs)
    rng = np.random.default_rng(4)
    sid = pool.create()
    h = {sid: c.create()}
    k = draw(rng, (L, 24, Hkv, D), "bf16")
    v = draw(rng, (L, 24, Hkv, D), "bf16")
    pool.append(sid, k.f32(), v.f32())            # context 20 tokens, then a 4-node tree
    c.append([h[sid]], [24], to_device(k), to_device(v))
    par = [-1, 0, 0, 2]
    for bad in ([1], [0, 0], [0, 4], [-1], [0, 1, 3]):
        with pytest.raises(pkv.PkvError) as e:
            c.commit(h[sid], par, bad)
        assert e.value.code == pkv.PKV_E_INVALID
    with pytest.raises(pkv.PkvError):             # parent after child
        c.commit(h[sid], [-1, 2, 0, 2], [0])
    with pytest.raises(pkv.PkvError):             # tree longer than the sequence
        c.commit(h[sid], [-1] + list(range(24)), [0])
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        binding.pkv_tree_commit(c.handle, h[sid], par, [0, 2], small)
    assert e.value.code == pkv.PKV_E_WORKSPACE
    same_state(c, h, pool, "after rejected commits")
    # a fork shares the partly filled second block; keeping node 0 needs a
    # copy of it and the pool has no free block
    fsid = pool.fork(sid)
    h[fsid] = c.fork(h[sid])
    with pytest.raises(oracle.OOMError):
        pool.commit(sid, 4, par, [0])
    with pytest.raises(pkv.OOM):
        c.commit(h[sid], par, [0])
    same_state(c, h, pool, "after an out-of-blocks commit")
    # freeing the fork makes room: the commit now goes through in place
    pool.free(fsid)
    c.free(h.pop(fsid))
    pool.commit(sid, 4, par, [0, 2, 3])
    c.commit(h[sid], par, [0, 2, 3])
    same_state(c, h, pool, "after the commit")
    c.close()


@pytest.mark.parametrize("w", COMMIT_CASES[:3], ids=lambda w: w.name)
def test_commit_batch_matches_oracle(pkv, w):
    """All requests of a verify step committed in one call (one random root
    path, one empty path, one deepest path, cycling), with a fork of the
    first request sharing its context tail: tables, counts and K/V bits
    equal the oracle's batch commit; decode afterwards agrees."""
    note(f"commit batch {w.name}")
    inp = generate(w)
    c, h = build_library(pkv, w, inp)
    pool = build_oracle(w, inp)
    reqs = list(w.query_sids)
    fsid = pool.fork(reqs[0])
    h[fsid] = c.fork(h[reqs[0]])
    rng = np.random.default_rng(6)
    N = w.n_nodes
    items = []
    for r, sid in enumerate(reqs):
        par = [int(x) for x in inp.parents[r]]
        if r % 3 == 1:
            path = []
        elif r % 3 == 2:
            depth = [len(root_path(par, j)) for j in range(N)]
            path = root_path(par, int(np.argmax(depth)))
        else:
            path = root_path(par, int(rng.integers(N)))
        items.append((sid, N, par, path))
    pool.commit_batch(items)
    c.commit_batch([h[sid] for sid in reqs], np.array([it[2] for it in items]),
                   [it[3] for it in items])
    same_state(c, h, pool, f"{w.name} after the batch")
    sh = w.shape
    live = [s for s in reqs + [fsid] if pool.length(s) > 0]
    q = draw(np.random.default_rng(10), (sh.L, len(live), sh.Hq, sh.D), "bf16")
    got = c.decode([h[s] for s in live], to_device(q), scale=w.softmax_scale)
    torch.cuda.synchronize()
    want = oracle.decode(pool, live, q.f32(), w.softmax_scale)
    check_close(got.cpu().numpy(), want, f"decode after batch commit {w.name}")
    c.close()


def test_commit_batch_out_of_blocks_changes_nothing(pkv):
    """The oracle's hand-built case on the device (block size 16): the first
    request alone would fit, the batch does not, and nothing changes."""
    L, Hkv, Hq, D, bs = 1, 1, 2, 64, 16
    c = pkv.PagedKVCache(4, bs, L, Hkv, Hq, D, dtype="bf16", device="cuda")
    pool = oracle.OraclePool(4, bs)
    rng = np.random.default_rng(12)
    h = {}

    def grow(sid, n):
        k = draw(rng, (L, n, Hkv, D), "bf16")
        v = draw(rng, (L, n, Hkv, D), "bf16")
        pool.append(sid, k.f32(), v.f32())
        c.append([h[sid]], [n], to_device(k), to_device(v))

    a = pool.create()
    h[a] = c.create()
    grow(a, 24)                                    # context: block 0, block 1 (8 of 16)
    grow(a, 8)                                     # tree: 8 nodes fill block 1
    b = pool.create()
    h[b] = c.create()
    grow(b, 8)                                     # context: block 2 (8 of 16)
    grow(b, 8)                                     # tree: 8 nodes fill block 2
    for s in (a, b):
        f = pool.fork(s)
        h[f] = c.fork(h[s])
    chain = [-1] + list(range(7))
    with pytest.raises(oracle.OOMError):
        pool.commit_batch([(a, 8, chain, [0]), (b, 8, chain, [0])])
    with pytest.raises(pkv.OOM):
        c.commit_batch([h[a], h[b]], np.array([chain, chain]), [[0], [0]])
    same_state(c, h, pool, "after the refused batch")
    pool.commit_batch([(a, 8, chain, [0, 1, 2])])
    c.commit_batch([h[a]], np.array([chain]), [[0, 1, 2]])
    same_state(c, h, pool, "after a alone")
    c.close()
