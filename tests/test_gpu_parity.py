"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Tables and K/V bytes: bit-exact. Attention outputs: max |error| <= 2e-3 and
relative L2 error <= 1e-2 against the oracle's float64 values (bf16 K/V,
fp32 arithmetic). The relative guard matters at long contexts, where
outputs are small (|o| ~ sqrt(e/N)) and 2e-3 alone would be loose.
"""

from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import configs, generate, get, scaled  # noqa: E402
from workloads.configs import replace_shape  # noqa: E402
from workloads.gen import Tensor, draw  # noqa: E402

from gpu_helpers import (arena_bits, build_library, build_oracle, errors, gather,  # noqa: E402
                         raw_bits, to_device)

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-3
REL_L2 = 1e-2


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_close(got, want, what):
    ma, rl = errors(got, want)
    note(f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e}")
    assert np.all(np.isfinite(got)), what
    assert ma <= MAX_ABS and rl <= REL_L2, (what, ma, rl)
    return ma, rl


B16 = configs.BEAM
AG = configs.AGENT

SMALL_DECODE = [
    get("tiny_a"),
    get("tiny_b"),
    scaled("beam", "beam_s", shape=replace_shape(B16, L=3, Hq=8, Hkv=2), root_len=200,
           n_branches=5, branch_len=37),
    scaled("mcts", "mcts_s", shape=replace_shape(B16, L=2, Hq=8, Hkv=2), root_len=100, depth=3,
           edge_len=21),
    scaled("agent", "agent_s", shape=replace_shape(AG, Hq=12, Hkv=2), root_len=300, n_branches=3,
           branch_len=170),
    scaled("beam_cow", "cow_d64", shape=replace_shape(B16, L=2, Hq=4, Hkv=1, D=64), root_len=40,
           n_branches=5, branch_len=3),
    scaled("beam", "bs64_d64", shape=replace_shape(B16, L=2, Hq=6, Hkv=3, D=64, BS=64), root_len=130,
           n_branches=3, branch_len=70),
    scaled("agent", "gqa1_d128_bs32", shape=replace_shape(AG, Hq=2, Hkv=2, D=128), root_len=33,
           n_branches=2, branch_len=1),
    # more than 32 query rows share the root and the first edges: wide items
    scaled("mcts", "mcts_wide", shape=replace_shape(B16, L=2, Hq=16, Hkv=2), root_len=77, depth=4,
           edge_len=19),
    scaled("beam", "beam_wide_d256", shape=replace_shape(AG, L=1, Hq=24, Hkv=2), root_len=150,
           n_branches=9, branch_len=40),
    # the tiny tree in bf16 too (the oracle reads the same rounded values)
    scaled("tiny_b", "tiny_b_bf16", shape=replace_shape(configs.TINY, dtype="bf16")),
]


PLAN = {}   # plan_info of the last run_decode call


def run_decode(w, path=0, chunk_tokens=0, order=None, rows_per_item=None, wide=1, prefetch=0,
               row_blocks=1, wide_shape=None, concurrent=0, short_items=1, short_tokens=256, fold=64,
               scale=None, inline_plan=1, group=16, spec=0):
    inp = generate(w)
    c, h = build_library(pytest.pkv, w, inp, alloc_order=order)
    c.set_option("inline_plan", inline_plan)
    c.set_option("wide_spec", spec)
    c.set_option("fold_tokens", fold)
    c.set_option("group_rows", group)
    c.set_option("concurrent", concurrent)
    c.set_option("short_items", short_items)
    c.set_option("short_tokens", short_tokens)
    if wide_shape:
        c.set_option("wide_waves", wide_shape[0])
        c.set_option("wide_row_blocks", wide_shape[1])
    c.set_option("path", path)
    c.set_option("prefetch", prefetch)
    c.set_option("row_blocks_per_wave", row_blocks)
    c.set_option("chunk_tokens", chunk_tokens)
    c.set_option("wide", wide)
    if rows_per_item:
        c.set_option("rows_per_item", rows_per_item)
    seqs = [h[s] for s in w.query_sids]
    q = to_device(inp.q)
    out = c.decode(seqs, q, scale=w.softmax_scale if scale is None else scale)
    torch.cuda.synchronize()
    res = out.cpu().numpy()
    PLAN.clear()
    PLAN.update(c.plan_info(seqs))
    c.close()
    return inp, res


@pytest.fixture(autouse=True, scope="module")
def _lib(pkv):
    pytest.pkv = pkv


@pytest.mark.parametrize("w", SMALL_DECODE, ids=lambda w: w.name)
@pytest.mark.parametrize("path,chunk,pf,rbw", [(0, 0, 0, 1), (0, 64, 0, 1), (0, 0, 0, 2), (0, 96, 1, 1),
                                              (1, 0, 0, 1), (1, 64, 0, 1), (0, 0, 0, 0)],
                         ids=["auto", "auto_split64", "two_blocks_per_wave", "prefetch_split96", "valu",
                              "valu_split64", "auto_blocks_per_wave"])
def test_decode_matches_oracle(w, path, chunk, pf, rbw):
    note(f"decode {w.name} path={path} chunk={chunk} prefetch={pf} row_blocks={rbw}")
    inp, got = run_decode(w, path=path, chunk_tokens=chunk, prefetch=pf, row_blocks=rbw)
    pool = build_oracle(w, inp)
    want = oracle.decode(pool, w.query_sids, inp.q.f32(), w.softmax_scale)
    check_close(got, want, f"{w.name} path={path} chunk={chunk}")


@pytest.mark.parametrize("w", [SMALL_DECODE[2], SMALL_DECODE[3], SMALL_DECODE[4]], ids=lambda w: w.name)
def test_page_layout_does_not_change_output(w):
    """A permuted allocation order moves every block; the plan depends only
    on the logical structure, so the output is bit-identical."""
    note(f"layout {w.name}")
    _, a = run_decode(w)
    order = np.random.default_rng(7).permutation(w.num_blocks_bound() + 8)
    _, b = run_decode(w, order=order)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("w", [SMALL_DECODE[2], SMALL_DECODE[4]], ids=lambda w: w.name)
def test_split_and_row_grouping_agree(w):
    note(f"splits {w.name}")
    inp, base = run_decode(w)
    for chunk, rpi, rbw in [(32, None, 1), (96, 16, 1), (0, 8, 1), (0, 48, 1), (0, 48, 2), (0, 64, 2)]:
        _, other = run_decode(w, chunk_tokens=chunk, rows_per_item=rpi, row_blocks=rbw)
        ma, _ = errors(other, base)
        assert ma <= 1e-4, (chunk, rpi, rbw, ma)


@pytest.mark.parametrize("w", [SMALL_DECODE[8], SMALL_DECODE[9]], ids=lambda w: w.name)
def test_wide_and_narrow_items_agree(w):
    """Rows of a chunk served by wide items (LDS-staged, two row blocks per
    wave) or by narrow ones give the same result to fp32 rounding."""
    note(f"wide/narrow {w.name}")
    inp, wide = run_decode(w, wide=1)
    _, narrow = run_decode(w, wide=0, rows_per_item=64)
    ma, _ = errors(wide, narrow)
    assert ma <= 1e-4, ma
    _, chunked = run_decode(w, wide=1, chunk_tokens=32)
    assert errors(chunked, wide)[0] <= 1e-4


@pytest.mark.parametrize("w", [SMALL_DECODE[2], SMALL_DECODE[3], SMALL_DECODE[4], SMALL_DECODE[8]],
                         ids=lambda w: w.name)
@pytest.mark.parametrize("chunk,pf,st", [(0, 0, 64), (0, 0, 256), (0, 0, 8192), (32, 0, 256),
                                         (32, 1, 256), (0, 1, 8192)])
def test_short_items_one_wave_each(w, chunk, pf, st):
    """Short narrow items (<= 16 rows, <= st tokens) run one (layer, head)
    plane per wave; the results match the four-wave form to fp32 rounding
    and the oracle to tolerance."""
    note(f"short items {w.name} chunk={chunk} prefetch={pf} short_tokens={st}")
    inp, a = run_decode(w, chunk_tokens=chunk, prefetch=pf, short_items=1, short_tokens=st)
    _, b = run_decode(w, chunk_tokens=chunk, prefetch=pf, short_items=0)
    assert errors(a, b)[0] <= 1e-4
    pool = build_oracle(w, inp)
    want = oracle.decode(pool, w.query_sids, inp.q.f32(), w.softmax_scale)
    check_close(a, want, f"{w.name} short items chunk={chunk}")


@pytest.mark.parametrize("w", [SMALL_DECODE[1], SMALL_DECODE[3], SMALL_DECODE[8]], ids=lambda w: w.name)
@pytest.mark.parametrize("fold", [0, 32, 64, 200])
def test_folded_short_segments_match_oracle(w, fold):
    """Short shared segments read per branch (folded into the branch's
    neighbouring short segments) give the oracle's outputs, and agree with
    the unfolded plan to fp32 rounding."""
    note(f"fold {w.name} fold_tokens={fold}")
    inp, a = run_decode(w, fold=fold)
    _, b = run_decode(w, fold=0)
    assert errors(a, b)[0] <= 1e-4
    pool = build_oracle(w, inp)
    want = oracle.decode(pool, w.query_sids, inp.q.f32(), w.softmax_scale)
    check_close(a, want, f"{w.name} fold_tokens={fold}")


GROUPED = [
    SMALL_DECODE[3],   # G 4: groups of 4 leaves; 21-token edges: each leaf's last block part-filled
    SMALL_DECODE[8],   # G 8: pairs of leaves, beside a wide root
    scaled("mcts", "mcts_d64_bs32", shape=replace_shape(B16, L=2, Hq=8, Hkv=2, D=64, BS=32),
           root_len=90, depth=4, edge_len=13),
    # 64-token edges fill whole 64-token blocks (folded with fold_tokens 128)
    scaled("mcts", "mcts_d256_bs64", shape=replace_shape(AG, L=1, Hq=8, Hkv=2, BS=64), root_len=100,
           depth=3, edge_len=64),
    scaled("mcts", "mcts_g1", shape=replace_shape(B16, L=1, Hq=2, Hkv=2), root_len=50, depth=5,
           edge_len=9),
]


@pytest.mark.parametrize("w", GROUPED, ids=lambda w: w.name)
@pytest.mark.parametrize("group,pf,st,chunk", [(16, 0, 256, 0), (8, 0, 256, 0), (16, 1, 256, 0),
                                               (16, 0, 8192, 0), (16, 0, 32, 0), (16, 0, 256, 64)],
                         ids=["rows16", "rows8", "prefetch", "one_wave", "four_waves", "split64"])
def test_grouped_siblings_match_oracle(w, group, pf, st, chunk):
    """Sibling leaves served by one item that reads their blocks once, each
    masked for the rows whose leaf does not hold it (option group_rows):
    the oracle's outputs, and the per-leaf plan's to fp32 rounding; on one
    wave or four (short_tokens), with the prefetching loop, and with each
    group cut into 64-token chunks (each chunk's slice of the block words,
    partial states and a combine)."""
    note(f"grouped {w.name} group_rows={group} prefetch={pf} short_tokens={st} chunk={chunk}")
    fold = 128 if w.shape.BS == 64 else 64
    inp, a = run_decode(w, group=group, prefetch=pf, short_tokens=st, fold=fold, chunk_tokens=chunk)
    grouped = PLAN["grouped_items"]
    G = w.shape.Hq // w.shape.Hkv
    # (pairs of the 21-token-edge tree share too little to be grouped)
    assert grouped > 0 if group == 16 else (grouped == 0 or group // G >= 2), (w.name, grouped)
    _, b = run_decode(w, group=0, prefetch=pf, short_tokens=st, fold=fold, chunk_tokens=chunk)
    assert PLAN["grouped_items"] == 0
    assert errors(a, b)[0] <= 1e-4
    pool = build_oracle(w, inp)
    want = oracle.decode(pool, w.query_sids, inp.q.f32(), w.softmax_scale)
    check_close(a, want, f"{w.name} grouped rows={group}")


def test_grouped_with_repeated_and_reordered_branches():
    """The batch of the 21-token-edge tree in reverse order with three leaves
    listed twice: groups follow the leaves' paths, not the batch order, and a
    repeated leaf is one more holder of the same blocks; the oracle's
    outputs, and the ungrouped plan's to fp32 rounding."""
    base = SMALL_DECODE[3]
    w = dataclasses.replace(base, name="mcts_s_repeated",
                            query_sids=tuple(reversed(base.query_sids)) + base.query_sids[:3])
    note(f"grouped {w.name}: {len(w.query_sids)} branches")
    inp, a = run_decode(w)
    assert PLAN["grouped_items"] > 0
    _, b = run_decode(w, group=0)
    assert errors(a, b)[0] <= 1e-4
    pool = build_oracle(w, inp)
    want = oracle.decode(pool, w.query_sids, inp.q.f32(), w.softmax_scale)
    check_close(a, want, f"{w.name} grouped")


def test_grouped_forks_with_unequal_valid_counts():
    """Forks of a 40-token root truncated to 40, 39, 38 and 37 tokens hold the
    root's third block (8 slots filled) with 8, 7, 6 and 5 valid slots: the
    group's item reads that block once per valid count, each for its own
    rows; two further forks add a block of their own. Against the oracle."""
    L, Hkv, Hq, D, bs = 2, 2, 8, 128, 16
    rng = np.random.default_rng(11)
    c = pytest.pkv.PagedKVCache(64, bs, L, Hkv, Hq, D, dtype="bf16", device="cuda")
    pool = oracle.OraclePool(64, bs)
    h = {}
    n = 40
    k, v = draw(rng, (L, n, Hkv, D), "bf16"), draw(rng, (L, n, Hkv, D), "bf16")
    a = pool.create()
    h[a] = c.create()
    pool.append(a, k.f32(), v.f32())
    c.append([h[a]], [n], to_device(k), to_device(v))
    sids = []
    for j in range(4):
        s = pool.fork(a)
        h[s] = c.fork(h[a])
        pool.truncate(s, n - j)
        c.truncate(h[s], n - j)
        sids.append(s)
    for j in range(2):
        s = pool.fork(a)
        h[s] = c.fork(h[a])
        k1, v1 = draw(rng, (L, 12, Hkv, D), "bf16"), draw(rng, (L, 12, Hkv, D), "bf16")
        pool.append(s, k1.f32(), v1.f32())
        c.append([h[s]], [12], to_device(k1), to_device(v1))
        sids.append(s)
    seqs = [h[s] for s in sids]
    info = c.plan_info(seqs)
    note(f"unequal valid counts: {info}")
    assert info["grouped_items"] >= 1
    q = draw(rng, (L, len(sids), Hq, D), "bf16")
    got = c.decode(seqs, to_device(q), scale=D ** -0.5).cpu().numpy()
    want = oracle.decode(pool, sids, q.f32(), D ** -0.5)
    check_close(got, want, "grouped forks with unequal valid counts")
    c.set_option("group_rows", 0)
    assert c.plan_info(seqs)["grouped_items"] == 0
    base = c.decode(seqs, to_device(q), scale=D ** -0.5).cpu().numpy()
    assert errors(got, base)[0] <= 1e-4
    c.close()


@pytest.mark.parametrize("w", [SMALL_DECODE[2], SMALL_DECODE[8]], ids=lambda w: w.name)
def test_concurrent_launches_bit_identical(w):
    """The wide launch on the library's second stream (forked from and joined
    into the caller's) computes exactly what it computes in order."""
    note(f"concurrent {w.name}")
    _, a = run_decode(w, rows_per_item=16, concurrent=1)
    _, b = run_decode(w, rows_per_item=16, concurrent=0)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


WIDE_SHAPES = [(8, 1), (6, 1), (4, 1), (4, 2), (8, 2)]


@pytest.mark.parametrize("w", [SMALL_DECODE[3], SMALL_DECODE[8], SMALL_DECODE[9]], ids=lambda w: w.name)
def test_final_rows_from_the_narrow_launch(w):
    """When every branch has one narrow chunk and the rest wide (MCTS-like
    trees: the root wide, each leaf's folded path narrow), the narrow launch
    merges the wide partial states and writes the outputs itself, with the
    combine's arithmetic: the outputs are bit-identical to the combine path
    (finalize 0) and meet the oracle bar."""
    inp = generate(w)
    outs = []
    for fin in (1, 0):
        c, h = build_library(pytest.pkv, w, inp)
        c.set_option("finalize", fin)
        seqs = [h[s] for s in w.query_sids]
        for k in ("combine",):
            c.timing_read(k)
        c.set_option("timing", 1)
        out = c.decode(seqs, to_device(inp.q), scale=w.softmax_scale)
        torch.cuda.synchronize()
        c.set_option("timing", 0)
        n_combine = c.timing_read("combine")[1]
        note(f"{w.name} finalize={fin}: combine launches {n_combine}")
        outs.append((out.cpu().numpy(), n_combine))
        c.close()
    (got, n1), (ref, n0) = outs
    assert n0 == 1
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), w.name
    pool = build_oracle(w, inp)
    want = oracle.decode(pool, w.query_sids, inp.q.f32(), w.softmax_scale)
    check_close(got, want, f"{w.name} final rows from the narrow launch (combine launches {n1})")


@pytest.mark.parametrize("rpi", [16, 12, 8])
def test_final_rows_with_other_item_sizes(rpi):
    """Final rows with other narrow item sizes on ragged chunks (G = 12):
    with 16 or 12 rows per item each tail is one narrow item and writes its
    rows; with 8 the tails go wide and the combine runs; either way the
    outputs are bit-identical to the combine path."""
    w = SMALL_DECODE[9]          # beam_wide_d256: G = 12, wide root, narrow tails
    inp = generate(w)
    outs = []
    for fin in (1, 0):
        c, h = build_library(pytest.pkv, w, inp)
        c.set_option("finalize", fin)
        c.set_option("rows_per_item", rpi)
        seqs = [h[s] for s in w.query_sids]
        c.timing_read("combine")
        c.set_option("timing", 1)
        out = c.decode(seqs, to_device(inp.q), scale=w.softmax_scale)
        torch.cuda.synchronize()
        c.set_option("timing", 0)
        outs.append((out.cpu().numpy(), c.timing_read("combine")[1]))
        c.close()
    (got, n1), (ref, n0) = outs
    # a tail's 12 rows are narrow only while they fit one item (rows above
    # rows_per_item go to wide items, so a narrow chunk is never split)
    assert (n1, n0) == ((0, 1) if rpi >= 12 else (1, 1)), (rpi, n1, n0)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), rpi
    outs = [got]
    pool = build_oracle(w, inp)
    want = oracle.decode(pool, w.query_sids, inp.q.f32(), w.softmax_scale)
    check_close(outs[0], want, f"final rows, rows_per_item {rpi}")


@pytest.mark.parametrize("w", [SMALL_DECODE[1], SMALL_DECODE[2], SMALL_DECODE[3], SMALL_DECODE[8],
                               SMALL_DECODE[9]], ids=lambda w: w.name)
def test_plan_in_launch_arguments(w):
    """A plan of at most 12,288 bytes travels in the kernel launches' own
    arguments (no upload before them); with inline_plan 0 the same plan is
    staged and copied into the workspace. The kernels read the same arrays
    either way: bit-identical outputs, which meet the oracle bar (fp32 on the
    VALU kernel, narrow, wide + combine, and wide + final rows from the
    narrow launch)."""
    inp = generate(w)
    c, h = build_library(pytest.pkv, w, inp)
    info = c.plan_info([h[s] for s in w.query_sids])
    c.close()
    note(f"{w.name}: plan {info['plan_bytes']} B")
    assert 0 < info["plan_bytes"] <= 12288
    _, got = run_decode(w, inline_plan=1)
    _, ref = run_decode(w, inline_plan=0)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), w.name
    pool = build_oracle(w, inp)
    want = oracle.decode(pool, w.query_sids, inp.q.f32(), w.softmax_scale)
    check_close(got, want, f"{w.name} plan in the launch arguments")


@pytest.mark.parametrize("w", [SMALL_DECODE[8], SMALL_DECODE[9]], ids=lambda w: w.name)
@pytest.mark.parametrize("shape", WIDE_SHAPES, ids=lambda s: f"{s[0]}w{s[1]}b")
def test_wide_shapes_match_oracle(w, shape):
    """Every compiled wide-kernel shape (waves per workgroup x row blocks
    per wave; the library falls back to the nearest one a head size has)."""
    note(f"wide shape {w.name} {shape}")
    inp, got = run_decode(w, wide_shape=shape)
    pool = build_oracle(w, inp)
    want = oracle.decode(pool, w.query_sids, inp.q.f32(), w.softmax_scale)
    check_close(got, want, f"{w.name} wide {shape}")


@pytest.mark.parametrize("w", [SMALL_DECODE[2], SMALL_DECODE[8], SMALL_DECODE[9]], ids=lambda w: w.name)
@pytest.mark.parametrize("factor", [-1.0, 0.0, 3.0])
def test_softmax_scale_sign_and_zero(w, factor):
    """A negative, zero or large softmax scale: the wide kernel folds the
    scale into the exponent (unscaled scores, the sign moved onto q), the
    narrow one scales the scores; both must match the oracle."""
    scale = factor * w.softmax_scale
    note(f"scale {w.name} {scale:+.4f}")
    inp, got = run_decode(w, scale=scale)
    pool = build_oracle(w, inp)
    want = oracle.decode(pool, w.query_sids, inp.q.f32(), scale)
    check_close(got, want, f"{w.name} scale {scale:+.4f}")


@pytest.mark.parametrize("name,keep_root", [("tiny_a", True), ("tiny_b", True), ("tiny_b", False)])
def test_cow_and_writes_bit_exact(name, keep_root):
    """Every live sequence, read through the library's table from the device
    arenas, holds exactly its materialised tokens; the root keeps its own
    tokens while the branches copy and append (a fork never changes the
    parent)."""
    w = get(name)
    inp = generate(w)
    c, h = build_library(pytest.pkv, w, inp, free_ops=not keep_root)
    pool = build_oracle(w, inp, free_ops=not keep_root)
    kb, vb = arena_bits(c.k_arena), arena_bits(c.v_arena)
    for sid in pool.live():
        K, V = gather(c, kb, vb, h[sid])
        Ko, Vo = pool.kv(sid)
        assert np.array_equal(K, raw_bits(Ko, w.shape.dtype)), sid
        assert np.array_equal(V, raw_bits(Vo, w.shape.dtype)), sid
    c.close()


@pytest.mark.parametrize("seed,dtype,bs", [(0, "bf16", 16), (1, "f32", 16), (2, "bf16", 32), (3, "bf16", 64)])
def test_random_traces_device_bit_exact(pkv, seed, dtype, bs):
    """Random create / fork / append / free traces with real K/V: tables and
    the bytes every live sequence reads equal the oracle's."""
    note(f"random device trace seed={seed} {dtype} bs={bs}")
    rng = np.random.default_rng(1000 + seed)
    L, Hkv, Hq, D = 2, 2, 4, 64
    nb = 400   # large enough that the trace never runs dry (OOM is tested on the host)
    order = rng.permutation(nb).tolist() if seed % 2 else None
    c = pkv.PagedKVCache(nb, bs, L, Hkv, Hq, D, dtype=dtype, device="cuda", alloc_order=order)
    pool = oracle.OraclePool(nb, bs, alloc_order=order)
    h = {}
    sh = configs.Shape(L=L, Hq=Hq, Hkv=Hkv, D=D, BS=bs, dtype=dtype)
    for step in range(120):
        act = int(rng.integers(5)) if h else 0
        if act == 0 and len(h) < 10:
            sid = pool.create()
            h[sid] = c.create()
        elif act == 1 and len(h) < 10:
            p = list(h)[rng.integers(len(h))]
            sid = pool.fork(p)
            h[sid] = c.fork(h[p])
        elif act in (2, 3):
            sids = list(rng.choice(list(h), size=min(len(h), int(rng.integers(1, 4))), replace=False))
            counts = [int(rng.integers(0, bs + 5)) for _ in sids]
            ks, vs = [], []
            for n in counts:
                k = draw(rng, (L, n, Hkv, D), dtype)
                v = draw(rng, (L, n, Hkv, D), dtype)
                ks.append(k)
                vs.append(v)
            for s, k, v in zip(sids, ks, vs):
                pool.append(int(s), k.f32(), v.f32())
            kcat = np.concatenate([k.raw for k in ks], axis=1)
            vcat = np.concatenate([v.raw for v in vs], axis=1)
            if sum(counts):
                c.append([h[int(s)] for s in sids], counts, to_device(Tensor(kcat, dtype)),
                         to_device(Tensor(vcat, dtype)))
        elif h:
            sid = list(h)[rng.integers(len(h))]
            pool.free(sid)
            c.free(h.pop(sid))
    torch.cuda.synchronize()
    kb, vb = arena_bits(c.k_arena), arena_bits(c.v_arena)
    checked = 0
    for sid in pool.live():
        assert c.table(h[sid]) == pool.table(sid)
        if pool.length(sid) == 0:
            continue
        K, V = gather(c, kb, vb, h[sid])
        Ko, Vo = pool.kv(sid)
        assert np.array_equal(K, raw_bits(Ko, dtype))
        assert np.array_equal(V, raw_bits(Vo, dtype))
        checked += 1
    assert checked > 0
    c.close()


# ------------------------------------------------------------------ verify

def run_verify(w, order=None, chunk_tokens=0, parents=None, wide_shape=None, scale=None,
               inline_plan=1, spec=0):
    inp = generate(w)
    if parents is not None:
        inp.parents = parents
    c, h = build_library(pytest.pkv, w, inp, alloc_order=order)
    c.set_option("inline_plan", inline_plan)
    c.set_option("wide_spec", spec)
    if wide_shape:
        c.set_option("wide_waves", wide_shape[0])
        c.set_option("wide_row_blocks", wide_shape[1])
    c.set_option("chunk_tokens", chunk_tokens)
    reqs = [h[s] for s in w.query_sids]
    out = c.verify(reqs, inp.parents, to_device(inp.q), scale=w.softmax_scale if scale is None else scale)
    torch.cuda.synchronize()
    res = out.cpu().numpy()
    c.close()
    return inp, res


SMALL_VERIFY = [
    scaled("verify", "verify_s", shape=replace_shape(AG, Hq=12, Hkv=2), n_req=2, ctx_len=200,
           n_nodes=13, max_depth=4),
    scaled("verify", "verify_d128_bs16", shape=replace_shape(B16, L=1, Hq=8, Hkv=2), n_req=3,
           ctx_len=77, n_nodes=48, max_depth=8),
    scaled("verify", "verify_64nodes", shape=replace_shape(AG, Hq=4, Hkv=1, D=64, BS=64), n_req=1,
           ctx_len=64, n_nodes=64, max_depth=64),
    scaled("verify", "verify_1node", shape=replace_shape(AG, Hq=6, Hkv=1, D=128), n_req=2, ctx_len=5,
           n_nodes=1, max_depth=1),
    scaled("verify", "verify_noctx", shape=replace_shape(AG, Hq=6, Hkv=3, D=128), n_req=2, ctx_len=0,
           n_nodes=20, max_depth=5),
]


@pytest.mark.parametrize("w", SMALL_VERIFY, ids=lambda w: w.name)
@pytest.mark.parametrize("chunk", [0, 64])
def test_verify_matches_oracle(w, chunk):
    note(f"verify {w.name} chunk={chunk}")
    inp, got = run_verify(w, chunk_tokens=chunk)
    pool = build_oracle(w, inp)
    want = oracle.verify(pool, w.query_sids, inp.parents, inp.q.f32(), w.softmax_scale)
    check_close(got, want, f"verify {w.name} chunk={chunk}")


@pytest.mark.parametrize("w", SMALL_VERIFY[:2], ids=lambda w: w.name)
def test_verify_plan_in_launch_arguments(w):
    """Verify with its plan in the launch arguments and staged: bit-identical
    outputs that meet the oracle bar."""
    inp, got = run_verify(w, inline_plan=1)
    _, ref = run_verify(w, inline_plan=0)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), w.name
    pool = build_oracle(w, inp)
    want = oracle.verify(pool, w.query_sids, inp.parents, inp.q.f32(), w.softmax_scale)
    check_close(got, want, f"verify {w.name} plan in the launch arguments")


@pytest.mark.parametrize("shape", WIDE_SHAPES, ids=lambda s: f"{s[0]}w{s[1]}b")
def test_verify_wide_shapes(shape):
    for w in (SMALL_VERIFY[0], SMALL_VERIFY[1], SMALL_VERIFY[2]):
        note(f"verify {w.name} wide {shape}")
        inp, got = run_verify(w, wide_shape=shape)
        pool = build_oracle(w, inp)
        want = oracle.verify(pool, w.query_sids, inp.parents, inp.q.f32(), w.softmax_scale)
        check_close(got, want, f"verify {w.name} wide {shape}")


@pytest.mark.parametrize("factor", [-1.0, 0.0])
def test_verify_scale_sign_and_zero(factor):
    """Draft-tree verify (the wide kernel, masked tree positions) with a
    negative or zero softmax scale."""
    for w in (SMALL_VERIFY[0], SMALL_VERIFY[1]):
        scale = factor * w.softmax_scale
        note(f"verify {w.name} scale {scale:+.4f}")
        inp, got = run_verify(w, scale=scale)
        pool = build_oracle(w, inp)
        want = oracle.verify(pool, w.query_sids, inp.parents, inp.q.f32(), scale)
        check_close(got, want, f"verify {w.name} scale {scale:+.4f}")


def test_verify_chain_and_star_trees():
    w = SMALL_VERIFY[0]
    N = w.n_nodes
    for name, par in [("chain", np.arange(N) - 1), ("star", np.full(N, -1))]:
        parents = np.stack([par] * len(w.query_sids)).astype(np.int32)
        inp, got = run_verify(w, parents=parents)
        pool = build_oracle(w, inp)
        want = oracle.verify(pool, w.query_sids, parents, inp.q.f32(), w.softmax_scale)
        check_close(got, want, f"verify {name}")


# ------------------------------------- wide kernel with specialised waves

SPEC_DECODE = [
    SMALL_DECODE[8],   # mcts_wide: a 128-row root (the kernel only when forced)
    # 32 leaves x G 8: a 256-row root of 301 tokens (ragged last step), 16-token blocks
    scaled("mcts", "mcts_spec_256rows", shape=replace_shape(B16, L=2, Hq=16, Hkv=2), root_len=301,
           depth=5, edge_len=19),
    # 64 leaves x G 4 at head_dim 64, 32-token blocks
    scaled("mcts", "mcts_spec_d64_bs32", shape=replace_shape(B16, L=2, Hq=8, Hkv=2, D=64, BS=32),
           root_len=90, depth=6, edge_len=13),
    # 13 beams x G 16 = 208 rows (three pairs hold a row past the item), 64-token blocks
    scaled("beam", "beam_spec_bs64", shape=replace_shape(B16, L=1, Hq=16, Hkv=1, BS=64), root_len=200,
           n_branches=13, branch_len=40),
]


@pytest.mark.parametrize("w", SPEC_DECODE, ids=lambda w: w.name)
@pytest.mark.parametrize("spec,chunk", [(1, 0), (2, 0), (2, 64)], ids=["auto", "forced", "forced_split64"])
def test_spec_wide_kernel_matches_oracle(w, spec, chunk):
    """Wide items on the kernel whose softmax and P.V run on separate waves:
    the oracle's outputs to tolerance, and the wide kernel's to fp32
    rounding."""
    note(f"spec decode {w.name} wide_spec={spec} chunk={chunk}")
    inp, got = run_decode(w, chunk_tokens=chunk, spec=spec)
    assert PLAN["n_items"] > 0
    pool = build_oracle(w, inp)
    want = oracle.decode(pool, w.query_sids, inp.q.f32(), w.softmax_scale)
    check_close(got, want, f"{w.name} wide_spec={spec} chunk={chunk}")
    _, ref = run_decode(w, chunk_tokens=chunk, spec=0)
    assert errors(got, ref)[0] <= 1e-4


VERIFY_SPEC = scaled("verify", "verify_spec_d128_64nodes", shape=replace_shape(B16, L=1, Hq=8, Hkv=2),
                     n_req=2, ctx_len=150, n_nodes=64, max_depth=64)


@pytest.mark.parametrize("w", [SMALL_VERIFY[1], SMALL_VERIFY[2], SMALL_VERIFY[4], VERIFY_SPEC],
                         ids=lambda w: w.name)
@pytest.mark.parametrize("chunk", [0, 64])
def test_spec_wide_kernel_verify(w, chunk):
    """Draft-tree verify (ancestor masks) on the kernel with specialised
    waves, forced for every wide item."""
    note(f"spec verify {w.name} chunk={chunk}")
    inp, got = run_verify(w, chunk_tokens=chunk, spec=2)
    pool = build_oracle(w, inp)
    want = oracle.verify(pool, w.query_sids, inp.parents, inp.q.f32(), w.softmax_scale)
    check_close(got, want, f"spec verify {w.name} chunk={chunk}")
    for factor in (-1.0, 0.0):
        scale = factor * w.softmax_scale
        inp, got = run_verify(w, chunk_tokens=chunk, spec=2, scale=scale)
        want = oracle.verify(pool, w.query_sids, inp.parents, inp.q.f32(), scale)
        check_close(got, want, f"spec verify {w.name} scale {scale:+.4f}")


# --------------------------------------------------------- errors, edges

def test_errors_are_reported(pkv):
    c = pkv.PagedKVCache(8, 16, 1, 1, 2, 64, dtype="bf16", device="cuda")
    s = c.create()
    q = torch.zeros((1, 1, 2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pkv.PkvError) as e:          # empty sequence
        c.decode([s], q)
    assert e.value.code == pkv.PKV_E_INVALID
    k = torch.zeros((1, 3, 1, 64), dtype=torch.bfloat16, device="cuda")
    c.append([s], [3], k, k)
    with pytest.raises(pkv.PkvError):               # layer range
        c.decode([s], q, layer0=1, n_layers=1)
    with pytest.raises(pkv.PkvError) as e:          # 65 tree nodes
        c.verify([s], np.full((1, 65), -1), torch.zeros((1, 65, 2, 64), dtype=torch.bfloat16,
                                                        device="cuda"))
    with pytest.raises(pkv.PkvError):               # bad parent pointer
        c.verify([s], np.array([[0, 0, 1]]), torch.zeros((1, 3, 2, 64), dtype=torch.bfloat16,
                                                          device="cuda"))
    from paged_kv_cache_amd import binding
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    out = torch.empty((1, 1, 2, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        binding.pkv_decode_attn(c.handle, [s], 0, 1, q, out, 0.1, small)
    assert e.value.code == pkv.PKV_E_WORKSPACE
    f = pkv.PagedKVCache(8, 16, 1, 1, 1, 64, dtype="f32", device="cuda")
    t = f.create()
    kf = torch.zeros((1, 2, 1, 64), dtype=torch.float32, device="cuda")
    f.append([t], [2], kf, kf)
    with pytest.raises(pkv.PkvError) as e:          # verify needs bf16
        f.verify([t], np.array([[-1]]), torch.zeros((1, 1, 1, 64), device="cuda"))
    assert e.value.code == pkv.PKV_E_UNSUPPORTED
    c.close()
    f.close()


def test_single_token_returns_its_value(pkv):
    c = pkv.PagedKVCache(4, 16, 2, 2, 6, 128, dtype="bf16", device="cuda")
    s = c.create()
    rng = np.random.default_rng(3)
    k = draw(rng, (2, 1, 2, 128), "bf16")
    v = draw(rng, (2, 1, 2, 128), "bf16")
    c.append([s], [1], to_device(k), to_device(v))
    q = to_device(draw(rng, (2, 1, 6, 128), "bf16"))
    out = c.decode([s, s], torch.cat([q, q], dim=1)).cpu().numpy()
    want = v.f32()[:, 0]                            # [L][Hkv][D]
    for l in range(2):
        for hh in range(6):
            assert np.array_equal(out[l, 0, hh], want[l, hh // 3])
            assert np.array_equal(out[l, 1, hh], want[l, hh // 3])
    c.close()


# ------------------------------------------------ full-size, sampled outputs

def sampled_decode(name, n_samples=48, seed=0, tree=0, spec=0):
    """The full-size decode: one whole layer (every branch and query head,
    drawn at random) and n_samples rows drawn from all layers, against the
    oracle's float64 values."""
    w = get(name)
    note(f"full-size {name} (tree {tree}, wide_spec {spec}): generating inputs")
    inp = generate(w)
    c, h = build_library(pytest.pkv, w, inp)
    c.set_option("tree", tree)
    c.set_option("wide_spec", spec)
    seqs = [h[s] for s in w.query_sids]
    q = to_device(inp.q)
    c.set_option("timing", 1)
    out = c.decode(seqs, q, scale=w.softmax_scale)
    torch.cuda.synchronize()
    c.set_option("timing", 0)
    n_tree = c.timing_read("attention_tree")[1]
    got = out.cpu().numpy()
    info = c.plan_info(seqs)
    c.close()
    note(f"full-size {name}: plan {info}")
    assert (n_tree > 0) == (tree > 0 and info["n_items"] == 0)
    pool = build_oracle(w, inp)
    rng = np.random.default_rng(seed)
    qf = inp.q.f32()
    L, B, Hq, D = got.shape
    layer = int(rng.integers(L))
    want = oracle.decode(pool, list(w.query_sids), qf, w.softmax_scale, layers=[layer])[0]
    check_close(got[layer], want, f"full-size {name}, layer {layer} ({B * Hq} rows)")
    gs, ws = [], []
    for _ in range(n_samples):
        l, b, hh = int(rng.integers(L)), int(rng.integers(B)), int(rng.integers(Hq))
        want = oracle.decode_one(pool, w.query_sids[b], qf[l, b, hh], l, hh, Hq, w.softmax_scale)
        gs.append(got[l, b, hh])
        ws.append(want)
    check_close(np.stack(gs), np.stack(ws), f"full-size {name} ({n_samples} sampled rows)")
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("name", ["beam", "mcts", "agent"])
def test_full_size_decode_sampled(name):
    sampled_decode(name)


def test_full_size_mcts_tree_launch():
    """The MCTS batch through the tree launch (option tree 1 selects it for
    this batch): one whole layer and sampled rows against the oracle."""
    sampled_decode("mcts", seed=3, tree=1)


def test_full_size_mcts_specialised_waves():
    """The MCTS root (256 rows x 4096 tokens per plane) on the kernel with
    separate softmax and P.V waves (option wide_spec 1 takes it for this
    batch): one whole layer and sampled rows against the oracle."""
    sampled_decode("mcts", seed=5, spec=1)


def test_full_size_verify_sampled():
    """One whole verify request (every node and query head) and sampled
    nodes of the others."""
    w = get("verify")
    note("full-size verify: generating inputs")
    inp = generate(w)
    c, h = build_library(pytest.pkv, w, inp)
    reqs = [h[s] for s in w.query_sids]
    out = c.verify(reqs, inp.parents, to_device(inp.q), scale=w.softmax_scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    c.close()
    pool = build_oracle(w, inp)
    qf = inp.q.f32()
    rng = np.random.default_rng(1)
    G = w.shape.G

    def want_node(r, i, g, K, V, ctx):
        idx = list(range(ctx)) + [ctx + j for j in oracle.ancestors(inp.parents[r], i)]
        return oracle.attention._softmax_attend(qf[r, i, g * G:(g + 1) * G], K[idx, g], V[idx, g],
                                                w.softmax_scale)

    whole = int(rng.integers(len(reqs)))
    K, V = pool.kv(w.query_sids[whole], layer=0)
    ctx = K.shape[0] - w.n_nodes
    gs = [got[whole, i, g * G:(g + 1) * G] for i in range(w.n_nodes) for g in range(w.shape.Hkv)]
    ws = [want_node(whole, i, g, K, V, ctx) for i in range(w.n_nodes) for g in range(w.shape.Hkv)]
    check_close(np.concatenate(gs), np.concatenate(ws),
                f"full-size verify, request {whole} ({w.n_nodes * w.shape.Hq} rows)")
    gs, ws = [], []
    for _ in range(24):
        r, i, g = int(rng.integers(len(reqs))), int(rng.integers(w.n_nodes)), int(rng.integers(w.shape.Hkv))
        K, V = pool.kv(w.query_sids[r], layer=0)
        ctx = K.shape[0] - w.n_nodes
        gs.append(got[r, i, g * G:(g + 1) * G])
        ws.append(want_node(r, i, g, K, V, ctx))
    check_close(np.concatenate(gs), np.concatenate(ws), "full-size verify (24 sampled nodes)")
    assert np.all(np.isfinite(got))


def test_full_size_beam_cow_bit_exact():
    w = get("beam_cow")
    inp = generate(w)
    c, h = build_library(pytest.pkv, w, inp, free_ops=False)
    pool = build_oracle(w, inp, free_ops=False)
    assert len(pool.cow_log) == 8
    kb, vb = arena_bits(c.k_arena), arena_bits(c.v_arena)
    for sid in pool.live():
        K, V = gather(c, kb, vb, h[sid])
        Ko, Vo = pool.kv(sid)
        assert np.array_equal(K, raw_bits(Ko, "bf16")) and np.array_equal(V, raw_bits(Vo, "bf16"))
    c.close()
