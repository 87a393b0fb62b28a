"""The tree launch (one workgroup per (layer, KV head) reading every chunk of
the batch once for all rows that hold it, tree.hip) against the oracle, on
small trees where it is forced (option "tree" 2; the full-size MCTS decode
through it, option "tree" 1, is checked in test_gpu_parity.py).

Tolerance as elsewhere: max |error| <= 2e-3 and relative L2 <= 1e-2 against
the oracle's float64 values; against the narrow / wide items' plan the two
agree to fp32 rounding (<= 1e-4)."""

from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import configs, generate, scaled  # noqa: E402
from workloads.configs import replace_shape  # noqa: E402
from workloads.gen import Tensor, bf16_round, draw  # noqa: E402

from gpu_helpers import build_library, build_oracle, errors, to_device  # noqa: E402

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-3
REL_L2 = 1e-2
B16 = configs.BEAM


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_close(got, want, what):
    ma, rl = errors(got, want)
    note(f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e}")
    assert np.all(np.isfinite(got)), what
    assert ma <= MAX_ABS and rl <= REL_L2, (what, ma, rl)


TREES = [
    scaled("mcts", "mcts_s", shape=replace_shape(B16, L=2, Hq=8, Hkv=2), root_len=100, depth=3,
           edge_len=21),
    scaled("mcts", "mcts_wide", shape=replace_shape(B16, L=2, Hq=16, Hkv=2), root_len=77, depth=4,
           edge_len=19),
    # 64 leaves x G = 4 = 256 rows: every wave's four blocks full
    scaled("mcts", "mcts_d6", shape=replace_shape(B16, L=2, Hq=8, Hkv=2), root_len=300, depth=6,
           edge_len=20),
    scaled("beam", "beam_s", shape=replace_shape(B16, L=3, Hq=8, Hkv=2), root_len=200, n_branches=5,
           branch_len=37),
    scaled("beam", "bs64_d64", shape=replace_shape(B16, L=2, Hq=6, Hkv=3, D=64, BS=64), root_len=130,
           n_branches=3, branch_len=70),
    scaled("agent", "gqa1_d128_bs32", shape=replace_shape(configs.AGENT, Hq=2, Hkv=2, D=128),
           root_len=33, n_branches=2, branch_len=1),
    scaled("mcts", "mcts_d64_bs32", shape=replace_shape(B16, L=1, Hq=16, Hkv=2, D=64, BS=32),
           root_len=600, depth=3, edge_len=45),
]


def run(pkv, w, tree=2, stages=5, piece=512, order=None, scale=None):
    inp = generate(w)
    c, h = build_library(pkv, w, inp, alloc_order=order)
    c.set_option("tree", tree)
    c.set_option("tree_stages", stages)
    c.set_option("tree_piece_tokens", piece)
    seqs = [h[s] for s in w.query_sids]
    c.set_option("timing", 1)
    out = c.decode(seqs, to_device(inp.q), scale=w.softmax_scale if scale is None else scale)
    torch.cuda.synchronize()
    c.set_option("timing", 0)
    n_tree = c.timing_read("attention_tree")[1]
    c.close()
    return inp, out.cpu().numpy(), n_tree


@pytest.mark.parametrize("w", TREES, ids=lambda w: w.name)
@pytest.mark.parametrize("stages,piece", [(5, 512), (4, 64), (6, 1024)])
def test_tree_matches_oracle(pkv, w, stages, piece):
    note(f"tree {w.name} stages={stages} piece={piece}")
    inp, got, n_tree = run(pkv, w, stages=stages, piece=piece)
    assert n_tree == 1, "the tree launch did not run"
    want = oracle.decode(build_oracle(w, inp), w.query_sids, inp.q.f32(), w.softmax_scale)
    check_close(got, want, f"tree {w.name}")
    _, items, n0 = run(pkv, w, tree=0)
    assert n0 == 0
    assert errors(got, items)[0] <= 1e-4


@pytest.mark.parametrize("factor", [-1.0, 0.0, 3.0])
def test_tree_scale_sign_and_zero(pkv, factor):
    for w in (TREES[1], TREES[4]):
        scale = factor * w.softmax_scale
        note(f"tree {w.name} scale {scale:+.4f}")
        inp, got, _ = run(pkv, w, scale=scale)
        want = oracle.decode(build_oracle(w, inp), w.query_sids, inp.q.f32(), scale)
        check_close(got, want, f"tree {w.name} scale {scale:+.4f}")


def test_tree_layout_does_not_change_output(pkv):
    """A permuted allocation order moves every block; the tree plan depends
    only on the logical structure, so the output is bit-identical."""
    w = TREES[2]
    _, a, _ = run(pkv, w)
    order = np.random.default_rng(7).permutation(w.num_blocks_bound() + 8)
    _, b, _ = run(pkv, w, order=order)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_tree_truncated_forks(pkv):
    """Forks cut back into a block their sibling fills further: the block is
    a chunk per holder (read up to each one's own length)."""
    L, Hkv, Hq, D, bs = 2, 2, 16, 128, 16
    rng = np.random.default_rng(9)
    c = pkv.PagedKVCache(64, bs, L, Hkv, Hq, D, dtype="bf16", device="cuda")
    c.set_option("tree", 2)
    pool = oracle.OraclePool(64, bs)
    h = {}
    k, v = draw(rng, (L, 200, Hkv, D), "bf16"), draw(rng, (L, 200, Hkv, D), "bf16")
    a = pool.create()
    h[a] = c.create()
    pool.append(a, k.f32(), v.f32())
    c.append([h[a]], [200], to_device(k), to_device(v))
    sids = [a]
    for j in range(9):
        s = pool.fork(a)
        h[s] = c.fork(h[a])
        pool.truncate(s, 199 - 3 * j)
        c.truncate(h[s], 199 - 3 * j)
        sids.append(s)
    q = draw(rng, (L, len(sids), Hq, D), "bf16")
    got = c.decode([h[s] for s in sids], to_device(q), scale=D ** -0.5).cpu().numpy()
    want = oracle.decode(pool, sids, q.f32(), D ** -0.5)
    check_close(got, want, "tree, truncated forks")
    c.close()


def test_tree_overflow_walks_again(pkv):
    """Keys 40x larger late in the root than early: for the workgroups that
    walk the chunks forwards, each row's reference (its first maximum) lies
    far below its true maximum and the probabilities overflow; those
    workgroups walk again with the true maxima. The outputs meet the oracle
    bar either way."""
    L, Hkv, Hq, D, bs = 2, 2, 8, 128, 16
    rng = np.random.default_rng(13)
    c = pkv.PagedKVCache(96, bs, L, Hkv, Hq, D, dtype="bf16", device="cuda")
    c.set_option("tree", 2)
    c.set_option("tree_piece_tokens", 64)
    pool = oracle.OraclePool(96, bs)
    raw_k = rng.standard_normal((L, 600, Hkv, D), dtype=np.float32)
    raw_k[:, 400:] *= 40.0
    k = Tensor(bf16_round(raw_k), "bf16")
    v = draw(rng, (L, 600, Hkv, D), "bf16")
    root = pool.create()
    hr = c.create()
    pool.append(root, k.f32(), v.f32())
    c.append([hr], [600], to_device(k), to_device(v))
    sids, hs = [], []
    for j in range(16):
        s = pool.fork(root)
        hh = c.fork(hr)
        kk, vv = draw(rng, (L, 5, Hkv, D), "bf16"), draw(rng, (L, 5, Hkv, D), "bf16")
        pool.append(s, kk.f32(), vv.f32())
        c.append([hh], [5], to_device(kk), to_device(vv))
        sids.append(s)
        hs.append(hh)
    q = draw(rng, (L, len(sids), Hq, D), "bf16")
    got = c.decode(hs, to_device(q), scale=D ** -0.5).cpu().numpy()
    want = oracle.decode(pool, sids, q.f32(), D ** -0.5)
    check_close(got, want, "tree, overflow walked again")
    c.close()
