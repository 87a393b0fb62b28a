"""Pins for the CPU oracle (CPU only).

The oracle is checked against things other than itself: torch's
scaled_dot_product_attention on sequences assembled straight from the trace,
hand-derived closed forms (tests/golden/), refcount invariants and
closed-form refcount histograms, and brute-force equivalences. A last group
plants mistakes in the oracle and checks that these pins catch them.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import attention as oatt
from oracle.pool import OraclePool, run_trace
from workloads import configs, generate, get, scaled
from workloads.configs import Shape, replace_shape

from helpers import assemble_sequences, kv_for_op, run_structure

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sdpa_decode(q_heads: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """torch SDPA in float64: q [Hq][D], K/V [len][Hkv][D] -> [Hq][D]."""
    qt = torch.from_numpy(np.asarray(q_heads, np.float64))[None, :, None, :]
    kt = torch.from_numpy(np.asarray(K, np.float64)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.asarray(V, np.float64)).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)
    return o[0, :, 0, :].numpy()


def build_oracle(w, inp):
    pool = OraclePool(w.num_blocks_bound() + 4, w.shape.BS)
    run_trace(pool, w.ops, kv_for_op(inp))
    return pool


# --------------------------------------------------------------------------
# decode vs torch SDPA on independently assembled sequences
# --------------------------------------------------------------------------

SMALL_DECODE = [
    get("tiny_a"),
    get("tiny_b"),
    scaled("beam", "beam_small", shape=replace_shape(configs.BEAM, L=2, Hq=8, Hkv=2, D=32),
           root_len=96, n_branches=3, branch_len=21),
    scaled("mcts", "mcts_small", shape=replace_shape(configs.BEAM, L=1, Hq=4, Hkv=2, D=16),
           root_len=40, depth=3, edge_len=5),
    scaled("agent", "agent_small", shape=replace_shape(configs.AGENT, Hq=6, Hkv=2, D=32, BS=8),
           root_len=37, n_branches=4, branch_len=19),
    scaled("beam_cow", "beam_cow_small", shape=replace_shape(configs.BEAM, L=2, Hq=4, Hkv=1, D=16),
           root_len=40, n_branches=5, branch_len=3),
]


@pytest.mark.parametrize("w", SMALL_DECODE, ids=lambda w: w.name)
def test_decode_matches_sdpa(w):
    inp = generate(w)
    pool = build_oracle(w, inp)
    got = oracle.decode(pool, w.query_sids, inp.q.f32(), w.softmax_scale)
    seqs = assemble_sequences(w, inp)
    q = inp.q.f32()
    for b, s in enumerate(w.query_sids):
        K, V = seqs[s]
        for l in range(w.shape.L):
            want = sdpa_decode(q[l, b], K[l], V[l], w.softmax_scale)
            np.testing.assert_allclose(got[l, b], want, rtol=1e-12, atol=1e-12)


def test_decode_one_matches_decode():
    w = SMALL_DECODE[2]
    inp = generate(w)
    pool = build_oracle(w, inp)
    full = oracle.decode(pool, w.query_sids, inp.q.f32(), w.softmax_scale)
    q = inp.q.f32()
    for (l, b, h) in [(0, 0, 0), (1, 2, 7), (1, 1, 3)]:
        one = oracle.decode_one(pool, w.query_sids[b], q[l, b, h], l, h, w.shape.Hq, w.softmax_scale)
        np.testing.assert_allclose(one, full[l, b, h], rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# hand-derived closed forms
# --------------------------------------------------------------------------

def _frac(s):
    return float(Fraction(s))


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "attention_closed_forms.json")))["cases"],
                         ids=lambda c: c["name"][:40])
def test_golden_closed_forms(case):
    K = np.array(case["K"], np.float64)          # [len][Hkv][D]
    V = np.array(case["V"], np.float64)
    q = np.array(case["q"], np.float64)           # [Hq][D]
    n, Hkv, D = K.shape
    pool = OraclePool(4, n)
    s = pool.create()
    pool.append(s, K[None], V[None])
    got = oracle.decode(pool, [s], q[None, None], case["scale"])[0, 0]
    want = np.array([[_frac(x) for x in row] for row in case["expected"]])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(11)
    K = rng.standard_normal((3, 1, 2, 8)).astype(np.float32)
    V = rng.standard_normal((3, 1, 2, 8)).astype(np.float32)
    pool = OraclePool(2, 16)
    s = pool.create()
    pool.append(s, K, V)
    q = rng.standard_normal((3, 1, 4, 8)) * 10
    out = oracle.decode(pool, [s], q, 0.35)
    for l in range(3):
        for h in range(4):
            np.testing.assert_array_equal(out[l, 0, h], V[l, 0, h // 2].astype(np.float64))


def test_zero_query_and_equal_keys_give_mean_of_v():
    rng = np.random.default_rng(12)
    n = 37
    V = rng.standard_normal((1, n, 1, 16)).astype(np.float32)
    K = rng.standard_normal((1, n, 1, 16)).astype(np.float32)
    pool = OraclePool(8, 8)
    s = pool.create()
    pool.append(s, K, V)
    out0 = oracle.decode(pool, [s], np.zeros((1, 1, 1, 16)), 1.0)[0, 0, 0]
    np.testing.assert_allclose(out0, V[0, :, 0].astype(np.float64).mean(axis=0), atol=1e-14)
    Keq = np.repeat(K[:, :1], n, axis=1)
    pool2 = OraclePool(8, 8)
    s2 = pool2.create()
    pool2.append(s2, Keq, V)
    out1 = oracle.decode(pool2, [s2], rng.standard_normal((1, 1, 1, 16)) * 5, 0.7)[0, 0, 0]
    np.testing.assert_allclose(out1, V[0, :, 0].astype(np.float64).mean(axis=0), atol=1e-14)


def test_fork_without_append_gives_parent_output():
    w = get("tiny_b")
    inp = generate(w)
    pool = build_oracle(w, inp)
    kid = pool.fork(w.query_sids[0])
    q = inp.q.f32()[:, :1]
    a = oracle.decode(pool, [w.query_sids[0]], q, 0.125)
    b = oracle.decode(pool, [kid], q, 0.125)
    np.testing.assert_array_equal(a, b)


def test_mha_when_heads_equal():
    rng = np.random.default_rng(13)
    K = rng.standard_normal((1, 20, 3, 8)).astype(np.float32)
    V = rng.standard_normal((1, 20, 3, 8)).astype(np.float32)
    pool = OraclePool(4, 8)
    s = pool.create()
    pool.append(s, K, V)
    q = rng.standard_normal((1, 1, 3, 8))
    out = oracle.decode(pool, [s], q, 0.3)[0, 0]
    for h in range(3):
        single = OraclePool(4, 8)
        t = single.create()
        single.append(t, K[:, :, h:h + 1], V[:, :, h:h + 1])
        np.testing.assert_array_equal(oracle.decode(single, [t], q[:, :, h:h + 1], 0.3)[0, 0, 0], out[h])


# --------------------------------------------------------------------------
# block tables: hand derivation, invariants, closed-form histograms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_a", "tiny_b"])
def test_tiny_tables_golden(name):
    gold = json.load(open(os.path.join(GOLDEN, "tiny_tables.json")))[name]
    w = get(name)
    pool = OraclePool(16, w.shape.BS)
    first_slots = None
    for op in w.ops:
        if op.kind == "create":
            pool.create(op.sid)
        elif op.kind == "fork":
            pool.fork(op.parent, op.sid)
        elif op.kind == "append":
            slots, _ = pool.append(op.sid, *(np.zeros((1, op.n, 1, 1), np.float32),) * 2)
            if op.sid == 1:
                first_slots = slots
        elif op.kind == "free":
            pool.free(op.sid)
    for s, t in gold["tables"].items():
        assert pool.table(int(s)) == t
    for b, c in gold["refcounts"].items():
        assert pool.refcount(int(b)) == c
    assert [list(x) for x in pool.cow_log] == gold["cow_ops"]
    assert first_slots == gold["first_branch_slots"]
    assert all(pool.refcount(b) == 0 for b in range(12, 16))


def histogram(pool):
    h = {}
    for b in range(pool.num_blocks):
        r = pool.refcount(b)
        if r:
            h[r] = h.get(r, 0) + 1
    return h


@pytest.mark.parametrize("name,want", [
    ("beam", {8: 128, 1: 128}),
    ("mcts", {64: 256, 32: 4, 16: 8, 8: 16, 4: 32, 2: 64, 1: 128}),
    ("agent", {4: 416, 1: 4096}),
    ("tiny_a", {4: 4, 1: 4}),
    ("verify", {1: 4 * 1026}),
])
def test_refcount_closed_forms(name, want):
    """beam: 128 prompt blocks held by 8 beams + 8 x 16 private blocks.
    mcts: the 256 root blocks are held by all 64 leaves; an edge of depth k
    (2**k of them, 2 blocks each) by 64 / 2**k leaves. agent: 416 shared
    blocks by 4 requests (75% fewer prefix blocks than 4 private copies)."""
    w = get(name)
    pool = OraclePool(w.num_blocks_bound(), w.shape.BS)
    run_structure(pool, w)
    assert histogram(pool) == want


def check_invariants(pool: OraclePool):
    counts = [0] * pool.num_blocks
    for s in pool.live():
        t = pool.table(s)
        assert len(t) == -(-pool.length(s) // pool.block_size)
        assert len(set(t)) == len(t)
        for b in t:
            counts[b] += 1
    for r in pool.entries.values():                              # prompt-cache references
        counts[r["block"]] += 1
        assert r["parent"] == -1 or r["parent"] in pool.entries
    assert counts == pool.ref                                    # I1
    used = {b for b in range(pool.num_blocks) if pool.ref[b] > 0}
    assert used.isdisjoint(pool.free_blocks)                     # I2
    assert used | pool.free_blocks == set(range(pool.num_blocks))


def random_trace_run(seed: int, nb: int, bs: int, steps: int):
    rng = np.random.default_rng(seed)
    order = rng.permutation(nb) if seed % 2 else None
    pool = OraclePool(nb, bs, alloc_order=order)
    live = []
    for _ in range(steps):
        act = rng.integers(4) if live else 0
        if act == 0:
            live.append(pool.create())
        elif act == 1:
            p = live[rng.integers(len(live))]
            before_t, before_l, before_m = pool.table(p), pool.length(p), list(pool.mat[p])
            live.append(pool.fork(p))
            assert pool.table(p) == before_t and pool.length(p) == before_l    # I5
            assert all(a is b for a, b in zip(pool.mat[p], before_m))
        elif act == 2:
            s = live[rng.integers(len(live))]
            n = int(rng.integers(0, 2 * bs + 3))
            k = np.full((1, n, 1, 1), float(s), np.float32)
            snap = (pool.table(s), dict(pool.lens), list(pool.ref), set(pool.free_blocks))
            others = {o: pool.table(o) for o in pool.live() if o != s}
            try:
                slots, cows = pool.append(s, k, k)
            except oracle.OOMError:
                assert (pool.table(s), dict(pool.lens), list(pool.ref), set(pool.free_blocks)) == snap
                continue
            for sl in slots:                                      # I4
                assert pool.refcount(sl // bs) == 1
            for o, t in others.items():                           # other sequences untouched
                assert pool.table(o) == t
            for src, dst, nv in cows:
                assert 0 < nv < bs and pool.refcount(dst) == 1
        else:
            s = live.pop(rng.integers(len(live)))
            pool.free(s)
        check_invariants(pool)
    for s in live:
        pool.free(s)
    assert all(r == 0 for r in pool.ref)                          # I3
    assert pool.free_blocks == set(range(nb))


@pytest.mark.parametrize("seed", range(12))
def test_random_traces_keep_invariants(seed):
    random_trace_run(seed, nb=24 + seed, bs=4 if seed % 3 else 16, steps=300)


def test_oom_is_atomic():
    pool = OraclePool(3, 4)
    s = pool.create()
    pool.append(s, *(np.zeros((1, 6, 1, 1), np.float32),) * 2)   # blocks 0, 1 (2 of 4 in block 1)
    c = pool.fork(s)
    snap = (pool.table(s), pool.table(c), list(pool.ref), set(pool.free_blocks))
    with pytest.raises(oracle.OOMError):                          # needs CoW + 1 fresh = 2 > 1 free
        pool.append(c, *(np.zeros((1, 4, 1, 1), np.float32),) * 2)
    assert (pool.table(s), pool.table(c), list(pool.ref), set(pool.free_blocks)) == snap
    pool.append(c, *(np.zeros((1, 2, 1, 1), np.float32),) * 2)    # CoW only: fits
    assert pool.table(c) == [0, 2] and pool.refcount(1) == 1


def test_materialised_sequences_follow_the_trace():
    w = SMALL_DECODE[3]
    inp = generate(w)
    pool = build_oracle(w, inp)
    seqs = assemble_sequences(w, inp)
    assert sorted(seqs) == pool.live()
    for s, (K, V) in seqs.items():
        k2, v2 = pool.kv(s)
        np.testing.assert_array_equal(k2, K)
        np.testing.assert_array_equal(v2, V)


# --------------------------------------------------------------------------
# verify
# --------------------------------------------------------------------------

def _verify_setup(ctx, N, parents_fn, seed=3, Hq=4, Hkv=2, D=16, R=2):
    rng = np.random.default_rng(seed)
    pool = OraclePool(64, 8)
    reqs, data = [], []
    for r in range(R):
        s = pool.create()
        K = rng.standard_normal((1, ctx + N, Hkv, D)).astype(np.float32)
        V = rng.standard_normal((1, ctx + N, Hkv, D)).astype(np.float32)
        pool.append(s, K[:, :ctx], V[:, :ctx])
        pool.append(s, K[:, ctx:], V[:, ctx:])
        reqs.append(s)
        data.append((K[0], V[0]))
    q = rng.standard_normal((R, N, Hq, D))
    parents = np.stack([parents_fn(N) for _ in range(R)])
    return pool, reqs, data, q, parents


def test_verify_chain_equals_causal_attention():
    ctx, N, scale = 13, 7, 0.3
    pool, reqs, data, q, parents = _verify_setup(ctx, N, lambda n: np.arange(n) - 1)
    got = oracle.verify(pool, reqs, parents, q, scale)
    for r, (K, V) in enumerate(data):
        # causal attention of the N draft rows over [context + draft]: row i sees
        # positions < ctx + i + 1
        qt = torch.from_numpy(q[r]).permute(1, 0, 2)[None]           # 1, Hq, N, D
        kt = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2)[None]
        vt = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2)[None]
        mask = torch.zeros(N, ctx + N, dtype=torch.bool)
        for i in range(N):
            mask[i, :ctx + i + 1] = True
        want = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=True)
        np.testing.assert_allclose(got[r], want[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_verify_star_sees_context_and_self():
    ctx, N, scale = 10, 5, 0.5
    pool, reqs, data, q, parents = _verify_setup(ctx, N, lambda n: np.full(n, -1))
    got = oracle.verify(pool, reqs, parents, q, scale)
    for r, (K, V) in enumerate(data):
        for i in range(N):
            idx = list(range(ctx)) + [ctx + i]
            want = sdpa_decode(q[r, i], K[idx], V[idx], scale)
            np.testing.assert_allclose(got[r, i], want, rtol=1e-12, atol=1e-12)


def test_verify_node_equals_decode_on_its_path():
    w = scaled("verify", "verify_small", shape=replace_shape(configs.AGENT, Hq=4, Hkv=2, D=16, BS=8),
               n_req=2, ctx_len=29, n_nodes=12, max_depth=4)
    inp = generate(w)
    pool = build_oracle(w, inp)
    q = inp.q.f32()
    got = oracle.verify(pool, w.query_sids, inp.parents, q, w.softmax_scale)
    seqs = assemble_sequences(w, inp)
    for r, s in enumerate(w.query_sids):
        K, V = seqs[s]
        ctx = K.shape[1] - w.n_nodes
        for i in range(w.n_nodes):
            path = []
            j = i
            while j != -1:
                path.append(j)
                j = int(inp.parents[r, j])
            path = path[::-1]
            dp = OraclePool(64, 8)
            t = dp.create()
            dp.append(t, K[:, :ctx], V[:, :ctx])
            dp.append(t, K[:, [ctx + j for j in path]], V[:, [ctx + j for j in path]])
            want = oracle.decode(dp, [t], q[r, i][None, None], w.softmax_scale)[0, 0]
            np.testing.assert_allclose(got[r, i], want, rtol=1e-12, atol=1e-13)


def test_verify_parents_are_best_first_and_bounded():
    from workloads import verify_parents
    for r in range(4):
        p = verify_parents(4, r, 48, 8)
        assert p[0] == -1
        for i in range(1, 48):
            assert 0 <= p[i] < i
            assert len(oracle.ancestors(p, i)) <= 8


# --------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# --------------------------------------------------------------------------

def _no_scale(Q, K, V, scale):
    return _orig_attend(Q, K, V, 1.0)


def _no_max_shift_wrong_sign(Q, K, V, scale):
    Q = np.asarray(Q, np.float64); K = np.asarray(K, np.float64); V = np.asarray(V, np.float64)
    x = -(Q @ K.T) * scale
    p = np.exp(x - x.max(axis=1, keepdims=True))
    return (p @ V) / p.sum(axis=1, keepdims=True)


def _drop_last_key(Q, K, V, scale):
    return _orig_attend(Q, K[:-1], V[:-1], scale) if len(K) > 1 else _orig_attend(Q, K, V, scale)


def _v_unnormalised(Q, K, V, scale):
    Q = np.asarray(Q, np.float64); K = np.asarray(K, np.float64); V = np.asarray(V, np.float64)
    x = (Q @ K.T) * scale
    p = np.exp(x - x.max(axis=1, keepdims=True))
    return p @ V


_orig_attend = oatt._softmax_attend


@pytest.mark.parametrize("mutant", [_no_scale, _no_max_shift_wrong_sign, _drop_last_key, _v_unnormalised],
                         ids=lambda f: f.__name__)
def test_planted_attention_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(oatt, "_softmax_attend", mutant)
    with pytest.raises(AssertionError):
        test_decode_matches_sdpa(SMALL_DECODE[0])


def test_planted_gqa_mapping_mistake_is_caught(monkeypatch):
    def wrong_decode(pool, sids, q, scale, layers=None):
        L, B, Hq, D = q.shape
        out = np.empty((L, B, Hq, D))
        for b, s in enumerate(sids):
            for l in range(L):
                K, V = pool.kv(s, layer=l)
                Hkv = K.shape[1]
                for h in range(Hq):
                    out[l, b, h] = _orig_attend(q[l, b, h][None], K[:, h % Hkv], V[:, h % Hkv], scale)[0]
        return out
    monkeypatch.setattr(oracle, "decode", wrong_decode)
    case = json.load(open(os.path.join(GOLDEN, "attention_closed_forms.json")))["cases"][2]
    with pytest.raises(AssertionError):
        test_golden_closed_forms(case)


def test_planted_cow_mistake_is_caught(monkeypatch):
    """A pool that writes into the shared tail instead of copying it."""
    orig_append = OraclePool.append

    def no_cow_append(self, sid, k, v):
        n = k.shape[1]
        if n == 0:
            return [], []
        t = self.tables[sid]
        slots = []
        for _ in range(n):
            pos = self.lens[sid]
            if pos % self.block_size == 0:
                t.append(self._alloc())
            slots.append(t[pos // self.block_size] * self.block_size + pos % self.block_size)
            self.lens[sid] = pos + 1
        return slots, []
    monkeypatch.setattr(OraclePool, "append", no_cow_append)
    with pytest.raises(AssertionError):
        test_tiny_tables_golden("tiny_b")
    monkeypatch.setattr(OraclePool, "append", orig_append)


def test_planted_verify_mask_mistake_is_caught(monkeypatch):
    """Ancestors without the node itself."""
    def no_self(parents, i):
        j = int(parents[i])
        res = []
        while j != -1:
            res.append(j)
            j = int(parents[j])
        return sorted(res) if res else [i]
    monkeypatch.setattr(oatt, "ancestors", no_self)
    with pytest.raises(AssertionError):
        test_verify_chain_equals_causal_attention()


# --------------------------------------------------------- commit (f2)

def _tree_request(seed, ctx, n_nodes, bs=4, L=2, Hkv=2, D=4, max_depth=8, nb=64):
    """A pool holding one request: ctx context tokens then an n_nodes draft
    tree (parents drawn as for the verify workload)."""
    from workloads.gen import verify_parents
    rng = np.random.default_rng(seed)
    pool = OraclePool(nb, bs)
    s = pool.create()
    kv = rng.standard_normal((2, L, ctx + n_nodes, Hkv, D)).astype(np.float32)
    if ctx:
        pool.append(s, kv[0][:, :ctx], kv[1][:, :ctx])
    pool.append(s, kv[0][:, ctx:], kv[1][:, ctx:])
    parents = verify_parents(seed, 0, n_nodes, max_depth)
    return pool, s, kv, [int(x) for x in parents]


def _root_path(parents, leaf):
    path = []
    while leaf != -1:
        path.append(leaf)
        leaf = parents[leaf]
    return path[::-1]


def test_commit_of_a_whole_chain_changes_nothing():
    """A chain tree accepted in full is already in path order."""
    pool, s, kv, _ = _tree_request(1, 9, 7)
    chain = [-1] + list(range(6))
    t0, refs0 = pool.table(s), list(pool.ref)
    k0, v0 = pool.kv(s)
    slots, cows = pool.commit(s, 7, chain, list(range(7)))
    k1, v1 = pool.kv(s)
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    assert pool.table(s) == t0 and pool.ref == refs0 and cows == []
    check_invariants(pool)


def test_commit_of_no_node_keeps_the_context():
    pool, s, kv, parents = _tree_request(2, 10, 9)
    free0 = len(pool.free_blocks)
    pool.commit(s, 9, parents, [])
    assert pool.length(s) == 10
    k, v = pool.kv(s)
    assert np.array_equal(k, kv[0][:, :10]) and np.array_equal(v, kv[1][:, :10])
    # 19 tokens in 5 blocks of 4 -> 10 tokens in 3 blocks
    assert len(pool.table(s)) == 3 and len(pool.free_blocks) == free0 + 2
    check_invariants(pool)


@pytest.mark.parametrize("seed", range(6))
def test_commit_equals_appending_the_path(seed):
    """Committing a root path gives, by value, the sequence built by
    appending the context and then the path's tokens ("speculation never
    changes the text")."""
    ctx, N = 5 + seed, 12
    pool, s, kv, parents = _tree_request(10 + seed, ctx, N)
    leaf = int(np.random.default_rng(seed).integers(N))
    path = _root_path(parents, leaf)
    pool.commit(s, N, parents, path)
    ref = OraclePool(64, 4)
    r = ref.create()
    ref.append(r, kv[0][:, :ctx], kv[1][:, :ctx])
    for a in path:
        ref.append(r, kv[0][:, ctx + a:ctx + a + 1], kv[1][:, ctx + a:ctx + a + 1])
    assert pool.length(s) == ref.length(r) == ctx + len(path)
    k1, v1 = pool.kv(s)
    k2, v2 = ref.kv(r)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    check_invariants(pool)


def test_commit_copies_a_shared_tail_and_leaves_the_fork():
    """A fork taken before the commit shares the context's partly filled
    block: the commit copies it (never writing an aliased block) and the
    fork still reads the whole tree."""
    pool, s, kv, parents = _tree_request(4, 6, 8)   # context ends inside block 1
    f = pool.fork(s)
    kf0, vf0 = pool.kv(f)
    path = _root_path(parents, 7)
    slots, cows = pool.commit(s, 8, parents, path)
    assert len(cows) == 1 and cows[0][2] == 6 % 4
    kf1, vf1 = pool.kv(f)
    assert np.array_equal(kf0, kf1) and np.array_equal(vf0, vf1)
    assert pool.table(f)[:2] != pool.table(s)[:2]
    check_invariants(pool)


def test_commit_rejects_a_non_chain_and_changes_nothing():
    pool, s, kv, parents = _tree_request(5, 4, 6)
    snap = (pool.table(s), list(pool.ref), pool.length(s))
    inner = next(a for a in range(6) if parents[a] != -1)
    for bad in ([inner], [0, 0], [0, 6], [-1]):     # not from a root, repeated, out of range
        with pytest.raises(Exception):
            pool.commit(s, 6, parents, bad)
        assert (pool.table(s), list(pool.ref), pool.length(s)) == snap


def test_truncate_then_reappend_restores_the_sequence():
    pool, s, kv, _ = _tree_request(6, 11, 5)
    k0, v0 = pool.kv(s)
    pool.truncate(s, 7)
    assert pool.length(s) == 7 and len(pool.table(s)) == 2
    pool.append(s, k0[:, 7:], v0[:, 7:])
    k1, v1 = pool.kv(s)
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    check_invariants(pool)


def test_commit_that_runs_out_of_blocks_changes_nothing():
    """The re-append must copy the context's shared, partly filled block; with
    no free block the commit fails and leaves tables and K/V as they were."""
    from oracle.pool import OOMError
    bs = 4
    pool = OraclePool(2, bs)
    s = pool.create()
    kv = np.random.default_rng(7).standard_normal((2, 1, 8, 1, 4)).astype(np.float32)
    pool.append(s, kv[0][:, :6], kv[1][:, :6])     # context: 6 tokens
    pool.append(s, kv[0][:, 6:], kv[1][:, 6:])     # tree: nodes 0, 1 (a chain)
    f = pool.fork(s)
    snap = (pool.table(s), pool.table(f), list(pool.ref), set(pool.free_blocks), pool.length(s))
    k0, v0 = pool.kv(s)
    with pytest.raises(OOMError):
        pool.commit(s, 2, [-1, 0], [0])
    assert (pool.table(s), pool.table(f), list(pool.ref), set(pool.free_blocks),
            pool.length(s)) == snap
    k1, v1 = pool.kv(s)
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    check_invariants(pool)


# ------------------------------------------------------ prompt cache (f3)

def _tok_pool(nb=32, bs=4, cap=None):
    pool = OraclePool(nb, bs)
    if cap is not None:
        pool.cache_capacity = cap
    return pool


def _grow(pool, sid, n, rng=None):
    """Append n tokens with K/V drawn from rng (zeros without one)."""
    if rng is None:
        k = np.zeros((1, n, 1, 2), np.float32)
        pool.append(sid, k, k)
        return
    kv = rng.standard_normal((2, 1, n, 1, 2)).astype(np.float32)
    pool.append(sid, kv[0], kv[1])


def _chain_tokens(pool, eid):
    out = []
    while eid != -1:
        r = pool.entries[eid]
        out = list(r["tokens"]) + out
        eid = r["parent"]
    return out


def test_match_is_the_longest_cached_prefix_by_brute_force():
    """After random inserts (and the evictions a small pool forces), a match
    returns exactly the longest cached token prefix of the query, found by
    spelling out every entry's chain."""
    rng = np.random.default_rng(0)
    bs = 2
    pool = _tok_pool(nb=40, bs=bs)
    seqs = {}
    for step in range(60):
        toks = [int(t) for t in rng.integers(0, 3, size=int(rng.integers(1, 12)))]
        try:
            sid, m = pool.cache_match(toks)
            _grow(pool, sid, len(toks) - m)
        except oracle.OOMError:
            continue
        pool.cache_insert(sid, toks)
        seqs[sid] = toks
        if len(seqs) > 3:
            victim = sorted(seqs)[int(rng.integers(len(seqs)))]
            pool.free(victim)
            del seqs[victim]
        check_invariants(pool)
        q = [int(t) for t in rng.integers(0, 3, size=int(rng.integers(0, 14)))]
        best, best_blocks = 0, []
        for e in pool.entries:
            spelled = _chain_tokens(pool, e)
            if len(spelled) > best and q[:len(spelled)] == spelled:
                best = len(spelled)
                chain, x = [], e
                while x != -1:
                    chain.append(pool.entries[x]["block"])
                    x = pool.entries[x]["parent"]
                best_blocks = chain[::-1]
        sid, m = pool.cache_match(q)
        assert m == best and pool.table(sid) == best_blocks
        pool.free(sid)


def test_resumed_sequence_equals_one_computed_in_full():
    """Match, then append only the unmatched tail: the sequence holds the
    same K/V, token for token, as one built by appending everything."""
    rng = np.random.default_rng(1)
    bs = 4
    pool = _tok_pool(nb=64, bs=bs)
    sys_prompt = list(range(100, 122))                    # 22 tokens: 5 full blocks + 2
    a = pool.create()
    kv = rng.standard_normal((2, 1, 30, 1, 2)).astype(np.float32)
    pool.append(a, kv[0][:, :22], kv[1][:, :22])
    assert pool.cache_insert(a, sys_prompt) == 5
    ka, va = pool.kv(a)
    b, m = pool.cache_match(sys_prompt + [7, 8, 9])
    assert m == 20 and pool.table(b) == pool.table(a)[:5]
    pool.append(b, kv[0][:, 20:25], kv[1][:, 20:25])  # the unmatched tail, recomputed
    full = pool.create()
    pool.append(full, kv[0][:, :25], kv[1][:, :25])
    kb, vb = pool.kv(b)
    kf, vf = pool.kv(full)
    assert np.array_equal(kb, kf) and np.array_equal(vb, vf)
    assert np.array_equal(kb[:, :22], ka) and np.array_equal(vb[:, :22], va)
    check_invariants(pool)


def test_parked_blocks_outlive_their_sequence():
    pool = _tok_pool(nb=8, bs=4)
    a = pool.create()
    _grow(pool, a, 10)
    assert pool.cache_insert(a, list(range(10))) == 2     # two full blocks
    blocks = pool.table(a)
    pool.free(a)
    assert pool.ref[blocks[0]] == pool.ref[blocks[1]] == 1 and blocks[2] in pool.free_blocks
    b, m = pool.cache_match(list(range(10)))
    assert m == 8 and pool.table(b) == blocks[:2]
    assert pool.ref[blocks[0]] == 2
    check_invariants(pool)


def test_eviction_order_by_hand():
    """bs 2, 6 blocks. A = tokens 1..4 (entries a1 -> a2, stamp 1), B = 5, 6
    (entry b1, stamp 2), then a match of 1, 2 re-stamps a1 (stamp 3). With A
    and B freed, four allocations evict a2 (oldest leaf), b1, then a1 (a
    leaf once a2 is gone), and the fourth takes the last free block."""
    pool = _tok_pool(nb=6, bs=2)
    a = pool.create()
    _grow(pool, a, 4)                       # blocks 0, 1
    b = pool.create()
    _grow(pool, b, 2)                       # block 2
    assert pool.cache_insert(a, [1, 2, 3, 4]) == 2
    assert pool.cache_insert(b, [5, 6]) == 1
    m, n = pool.cache_match([1, 2, 9])
    assert n == 2 and pool.table(m) == [0]
    pool.free(m)
    pool.free(a)
    pool.free(b)
    assert sorted(pool.free_blocks) == [3, 4, 5] and pool.evictable() == 3
    c = pool.create()
    _grow(pool, c, 6)                       # takes 3, 4, 5: no eviction
    assert pool.table(c) == [3, 4, 5] and len(pool.entries) == 3
    _grow(pool, c, 2)                       # evicts a2 -> block 1
    assert pool.table(c)[-1] == 1 and len(pool.entries) == 2
    _grow(pool, c, 2)                       # evicts b1 -> block 2
    assert pool.table(c)[-1] == 2
    _grow(pool, c, 2)                       # evicts a1 -> block 0
    assert pool.table(c)[-1] == 0 and not pool.entries
    with pytest.raises(oracle.OOMError):
        _grow(pool, c, 1)
    check_invariants(pool)


def test_blocks_in_use_are_never_evicted():
    pool = _tok_pool(nb=4, bs=2)
    a = pool.create()
    _grow(pool, a, 4)
    pool.cache_insert(a, [1, 2, 3, 4])      # a still holds both blocks
    b = pool.create()
    _grow(pool, b, 4)                       # blocks 2, 3
    assert pool.evictable() == 0
    snap = (pool.table(a), pool.table(b), list(pool.ref), set(pool.free_blocks), len(pool.entries))
    with pytest.raises(oracle.OOMError):
        _grow(pool, b, 1)
    assert (pool.table(a), pool.table(b), list(pool.ref), set(pool.free_blocks),
            len(pool.entries)) == snap
    pool.free(a)                            # now both entries can go, leaf first
    assert pool.evictable() == 2
    _grow(pool, b, 1)
    assert pool.table(b)[-1] == 1 and len(pool.entries) == 1
    check_invariants(pool)


def test_capacity_stops_an_insert_and_spares_its_own_chain():
    pool = _tok_pool(nb=16, bs=2, cap=2)
    a = pool.create()
    _grow(pool, a, 6)
    assert pool.cache_insert(a, [1, 2, 3, 4, 5, 6]) == 2  # third block: nothing to evict
    pool.free(a)                                          # block 2 goes back to the free list
    b = pool.create()
    _grow(pool, b, 2)                                     # and b takes it
    assert pool.cache_insert(b, [7, 8]) == 1              # evicts the older leaf (block 1)
    assert sorted(r["block"] for r in pool.entries.values()) == [0, 2]
    _, n = pool.cache_match([1, 2, 3, 4])
    assert n == 2
    check_invariants(pool)


def test_insert_refreshes_existing_entries_and_clear_releases_all():
    pool = _tok_pool(nb=16, bs=2)
    a = pool.create()
    _grow(pool, a, 4)
    b = pool.fork(a)
    assert pool.cache_insert(a, [1, 2, 3, 4]) == 2
    assert pool.cache_insert(b, [1, 2, 3, 4]) == 0        # same keys: refreshed, not added
    assert pool.ref[pool.table(a)[0]] == 3
    pool.cache_clear()
    assert not pool.entries and pool.ref[pool.table(a)[0]] == 2
    with pytest.raises(oracle.InvalidError):
        pool.cache_insert(a, [1, 2, 3, 4, 5])             # more ids than tokens
    check_invariants(pool)


def test_commit_batch_equals_commits_by_value():
    """A batch of commits leaves every request with the same K/V as
    committing them one at a time; a batch of one is a commit exactly."""
    for seed in range(4):
        pools = []
        for _ in range(2):
            rng = np.random.default_rng(50 + seed)
            pool = OraclePool(96, 4)
            root = pool.create()
            ctx = int(rng.integers(3, 14))
            kv = rng.standard_normal((2, 1, ctx, 1, 4)).astype(np.float32)
            pool.append(root, kv[0], kv[1])
            reqs = [pool.fork(root) for _ in range(3)]
            trees = []
            for r in reqs:
                n = int(rng.integers(1, 10))
                t = rng.standard_normal((2, 1, n, 1, 4)).astype(np.float32)
                pool.append(r, t[0], t[1])
                par = [-1] + [int(rng.integers(-1, j)) for j in range(1, n)]
                trees.append((r, n, par, _root_path(par, int(rng.integers(n)))))
            pools.append((pool, trees))
        (a, trees), (b, _) = pools
        a.commit_batch(trees)
        for r, n, par, acc in trees:
            b.commit(r, n, par, acc)
        for r, *_ in trees:
            ka, va = a.kv(r)
            kb, vb = b.kv(r)
            assert np.array_equal(ka, kb) and np.array_equal(va, vb)
        check_invariants(a)
    pool, s, kv, parents = _tree_request(8, 7, 9)
    twin, s2, _, _ = _tree_request(8, 7, 9)
    path = _root_path(parents, 8)
    pool.commit_batch([(s, 9, parents, path)])
    twin.commit(s2, 9, parents, path)
    assert pool.table(s) == twin.table(s2) and pool.ref == twin.ref


def test_commit_batch_out_of_blocks_changes_nothing():
    """Requests a and b each keep one node; forks taken after their trees
    share both context tails, so each re-append must copy its tail. One
    block is free: a alone would fit, the batch does not, and the batch
    leaves a untouched too."""
    from oracle.pool import OOMError
    pool = OraclePool(4, 4)
    z = np.zeros((1, 8, 1, 2), np.float32)
    a = pool.create()
    pool.append(a, z[:, :6], z[:, :6])                     # context: blocks 0, 1 (2 of 4)
    pool.append(a, z[:, :2], z[:, :2])                     # tree: 2 nodes, fills block 1
    b = pool.create()
    pool.append(b, z[:, :2], z[:, :2])                     # context: block 2 (2 of 4)
    pool.append(b, z[:, :2], z[:, :2])                     # tree: 2 nodes, fills block 2
    fa, fb = pool.fork(a), pool.fork(b)
    assert sorted(pool.free_blocks) == [3]
    state = lambda: (pool.table(a), pool.table(b), pool.length(a), pool.length(b),
                     list(pool.ref), set(pool.free_blocks))
    snap = state()
    with pytest.raises(OOMError):
        pool.commit_batch([(a, 2, [-1, 0], [0]), (b, 2, [-1, 0], [0])])
    assert state() == snap
    pool.commit_batch([(a, 2, [-1, 0], [0])])              # alone, a fits
    assert pool.length(a) == 7 and pool.table(a)[1] == 3
    check_invariants(pool)
