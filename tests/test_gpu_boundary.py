"""Device tests of the boundary's standalone table-to-device calls, of
appends and decodes after a truncate, and of the rule that a branch's output
does not depend on what runs beside it.

* pkv_seq_append_plan -> pkv_cow_copy -> pkv_write_kv, called one by one
  through the C ABI with real K/V: every live sequence, gathered through the
  library's table from the device arenas, equals the oracle's materialised
  sequence bit for bit (a fork is a shallow copy, a written block is never
  aliased: Dendrite author's replies, "How is this different from vLLM's
  paged attention?" and "Why Rust?").
* After a truncate, one block can hold 8 valid slots for one holder and 4
  for its truncated fork. When both append in one batch, the longer holder
  copies the block while the shorter one writes into it in place: the copy
  must read the block before the write lands.
* A request's output does not depend on what else is running (Ferrite
  page, section 06): each branch decoded alone and inside its batch meets
  the oracle bar both ways, and a branch decoded alone twice is
  bit-identical.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import configs, generate, get, scaled  # noqa: E402
from workloads.configs import replace_shape  # noqa: E402
from workloads.gen import Tensor, draw  # noqa: E402

from gpu_helpers import arena_bits, build_library, build_oracle, errors, gather, raw_bits, to_device  # noqa: E402

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


def check_bytes(c, pool, h, dtype):
    kb, vb = arena_bits(c.k_arena), arena_bits(c.v_arena)
    n = 0
    for sid in pool.live():
        assert c.table(h[sid]) == pool.table(sid), sid
        if pool.length(sid) == 0:
            continue
        K, V = gather(c, kb, vb, h[sid])
        Ko, Vo = pool.kv(sid)
        assert np.array_equal(K, raw_bits(Ko, dtype)), sid
        assert np.array_equal(V, raw_bits(Vo, dtype)), sid
        n += 1
    assert n > 0


STANDALONE = [
    get("tiny_b"),
    scaled("beam_cow", "beam_cow_s", shape=replace_shape(B16, L=3, Hq=8, Hkv=2), root_len=72,
           n_branches=5, branch_len=11),
    scaled("beam_cow", "beam_cow_bs32_f32", shape=replace_shape(B16, L=2, Hq=4, Hkv=2, D=64, BS=32,
                                                                dtype="f32"),
           root_len=45, n_branches=3, branch_len=40),
]


@pytest.mark.parametrize("w", STANDALONE, ids=lambda w: w.name)
def test_plan_copy_write_calls_bit_exact(pkv, w):
    """The trace driven through the three standalone calls instead of the
    fused append: plan (host), then the copy-on-write copy and the token
    writes as their own launches."""
    from paged_kv_cache_amd import binding
    note(f"standalone plan/copy/write {w.name}")
    inp = generate(w)
    sh = w.shape
    c = pkv.PagedKVCache(w.num_blocks_bound() + 8, sh.BS, sh.L, sh.Hkv, sh.Hq, sh.D,
                         dtype=sh.dtype, device="cuda")
    kv = {i: (k, v) for i, _sid, k, v in inp.appends}
    h, copies = {}, []
    for i, op in enumerate(w.ops):
        if op.kind == "create":
            h[op.sid] = c.create()
        elif op.kind == "fork":
            h[op.sid] = c.fork(h[op.parent])
        elif op.kind == "append":
            slots, cows = binding.pkv_seq_append_plan(c.handle, h[op.sid], op.n)
            if cows:
                binding.pkv_cow_copy(c.handle, cows)
                copies += cows
            k, v = kv[i]
            binding.pkv_write_kv(c.handle, slots, to_device(k), to_device(v))
        elif op.kind == "free":
            c.free(h.pop(op.sid))
    torch.cuda.synchronize()
    pool = build_oracle(w, inp)
    assert [tuple(x) for x in pool.cow_log] == copies and copies
    check_bytes(c, pool, h, sh.dtype)
    c.close()


def test_copy_calls_move_only_valid_slots(pkv):
    """pkv_cow_copy alone: the destination's slots [0, n_valid) of every
    layer and KV head, K and V, equal the source's; the source is unchanged."""
    from paged_kv_cache_amd import binding
    L, Hkv, D, BS = 2, 3, 128, 16
    c = pkv.PagedKVCache(8, BS, L, Hkv, Hkv, D, dtype="bf16", device="cuda")
    rng = np.random.default_rng(11)
    fill = draw(rng, (L, 8 * BS, Hkv, D), "bf16")
    s = c.create()
    c.append([s], [8 * BS], to_device(fill), to_device(draw(rng, (L, 8 * BS, Hkv, D), "bf16")))
    torch.cuda.synchronize()
    kb0, vb0 = arena_bits(c.k_arena), arena_bits(c.v_arena)
    binding.pkv_cow_copy(c.handle, [(1, 5, 9), (2, 6, 16), (3, 7, 1)])
    torch.cuda.synchronize()
    kb, vb = arena_bits(c.k_arena), arena_bits(c.v_arena)
    for src, dst, nv in [(1, 5, 9), (2, 6, 16), (3, 7, 1)]:
        assert np.array_equal(kb[:, dst, :, :nv], kb0[:, src, :, :nv])
        assert np.array_equal(vb[:, dst, :, :, :nv], vb0[:, src, :, :, :nv])
    for b in range(5):
        assert np.array_equal(kb[:, b], kb0[:, b]) and np.array_equal(vb[:, b], vb0[:, b])
    c.close()


@pytest.mark.parametrize("dtype,bs,first", [("bf16", 16, "long"), ("bf16", 16, "short"),
                                            ("f32", 32, "long"), ("bf16", 64, "long")])
def test_append_after_truncate_bit_exact(pkv, dtype, bs, first):
    """A holds 2.5 blocks; B = fork(A) is cut back into A's last block. Both
    append one token in one batch call. With A first, A copies the shared
    block and B (now its only holder) writes in place at an offset A's copy
    reads: the library must order the copy before the write. With B first, B
    copies and A writes in place. Either way the bytes equal the oracle's,
    and decoding A and B side by side meets the oracle bar."""
    note(f"append after truncate {dtype} bs={bs} {first} first")
    L, Hkv, Hq, D = 2, 2, 4, 64
    rng = np.random.default_rng(77 + bs)
    c = pkv.PagedKVCache(16, bs, L, Hkv, Hq, D, dtype=dtype, device="cuda")
    pool = oracle.OraclePool(16, bs)
    h = {}
    n_a = 2 * bs + bs // 2
    ka, va = draw(rng, (L, n_a, Hkv, D), dtype), draw(rng, (L, n_a, Hkv, D), dtype)
    a = pool.create()
    h[a] = c.create()
    pool.append(a, ka.f32(), va.f32())
    c.append([h[a]], [n_a], to_device(ka), to_device(va))
    b = pool.fork(a)
    h[b] = c.fork(h[a])
    cut = n_a - bs // 4
    pool.truncate(b, cut)
    c.truncate(h[b], cut)
    order = [a, b] if first == "long" else [b, a]
    ks = [draw(rng, (L, 1, Hkv, D), dtype) for _ in order]
    vs = [draw(rng, (L, 1, Hkv, D), dtype) for _ in order]
    for s, k, v in zip(order, ks, vs):
        pool.append(s, k.f32(), v.f32())
    kcat = Tensor(np.concatenate([k.raw for k in ks], axis=1), dtype)
    vcat = Tensor(np.concatenate([v.raw for v in vs], axis=1), dtype)
    c.append([h[s] for s in order], [1, 1], to_device(kcat), to_device(vcat))
    torch.cuda.synchronize()
    assert len(pool.cow_log) == 1
    check_bytes(c, pool, h, dtype)
    # decode both, side by side (the block B wrote in place is A's old tail)
    q = draw(rng, (L, 2, Hq, D), dtype)
    scale = D ** -0.5
    got = c.decode([h[a], h[b]], to_device(q), scale=scale).cpu().numpy()
    want = oracle.decode(pool, [a, b], q.f32(), scale)
    check_close(got, want, f"decode after truncate ({first} first)")
    c.close()


def test_decode_truncated_fork_beside_its_sibling(pkv):
    """A truncated fork still shares a partly filled block with its sibling,
    which holds more of it; the planner reads that block for each holder up
    to its own length. Checked against the oracle on narrow and wide items
    (many forks make the shared prefix wide)."""
    L, Hkv, Hq, D, bs = 2, 2, 16, 128, 16
    rng = np.random.default_rng(5)
    for n_forks in (1, 3, 9):
        note(f"truncated forks beside their sibling: {n_forks}")
        c = pkv.PagedKVCache(64, bs, L, Hkv, Hq, D, dtype="bf16", device="cuda")
        pool = oracle.OraclePool(64, bs)
        h = {}
        n = 200
        k, v = draw(rng, (L, n, Hkv, D), "bf16"), draw(rng, (L, n, Hkv, D), "bf16")
        a = pool.create()
        h[a] = c.create()
        pool.append(a, k.f32(), v.f32())
        c.append([h[a]], [n], to_device(k), to_device(v))
        sids = [a]
        for j in range(n_forks):
            s = pool.fork(a)
            h[s] = c.fork(h[a])
            cut = n - 1 - 3 * j
            pool.truncate(s, cut)
            c.truncate(h[s], cut)
            sids.append(s)
        q = draw(rng, (L, len(sids), Hq, D), "bf16")
        got = c.decode([h[s] for s in sids], to_device(q), scale=D ** -0.5).cpu().numpy()
        want = oracle.decode(pool, sids, q.f32(), D ** -0.5)
        check_close(got, want, f"{n_forks} truncated forks")
        c.close()


@pytest.mark.parametrize("seed,dtype,bs", [(0, "bf16", 16), (1, "f32", 16), (2, "bf16", 32),
                                           (3, "bf16", 16)])
def test_random_traces_with_truncate_device(pkv, seed, dtype, bs):
    """Random create / fork / truncate / batch-append / free traces with real
    K/V (truncates make holders of one block disagree on its valid count, so
    batch appends hit the copy-then-write-in-place case): tables and bytes
    equal the oracle's, and a decode of every live sequence meets the
    oracle bar."""
    note(f"random device trace with truncate seed={seed} {dtype} bs={bs}")
    rng = np.random.default_rng(2000 + seed)
    L, Hkv, Hq, D = 2, 2, 4, 64
    nb = 400
    c = pkv.PagedKVCache(nb, bs, L, Hkv, Hq, D, dtype=dtype, device="cuda")
    pool = oracle.OraclePool(nb, bs)
    h = {}
    for step in range(150):
        act = int(rng.integers(6)) if h else 0
        if act == 0 and len(h) < 10:
            sid = pool.create()
            h[sid] = c.create()
        elif act == 1 and len(h) < 10:
            p = list(h)[rng.integers(len(h))]
            sid = pool.fork(p)
            h[sid] = c.fork(h[p])
        elif act in (2, 3):
            sids = list(rng.choice(list(h), size=min(len(h), int(rng.integers(1, 5))), replace=False))
            counts = [int(rng.integers(0, bs + 5)) for _ in sids]
            ks = [draw(rng, (L, n, Hkv, D), dtype) for n in counts]
            vs = [draw(rng, (L, n, Hkv, D), dtype) for n in counts]
            for s, k, v in zip(sids, ks, vs):
                pool.append(int(s), k.f32(), v.f32())
            if sum(counts):
                kcat = Tensor(np.concatenate([k.raw for k in ks], axis=1), dtype)
                vcat = Tensor(np.concatenate([v.raw for v in vs], axis=1), dtype)
                c.append([h[int(s)] for s in sids], counts, to_device(kcat), to_device(vcat))
        elif act == 4:
            sid = list(h)[rng.integers(len(h))]
            m = int(rng.integers(0, pool.length(sid) + 1))
            pool.truncate(sid, m)
            c.truncate(h[sid], m)
        elif len(h) > 1:
            sid = list(h)[rng.integers(len(h))]
            pool.free(sid)
            c.free(h.pop(sid))
    torch.cuda.synchronize()
    check_bytes(c, pool, h, dtype)
    live = [s for s in pool.live() if pool.length(s) > 0]
    q = draw(rng, (L, len(live), Hq, D), dtype)
    got = c.decode([h[s] for s in live], to_device(q), scale=D ** -0.5).cpu().numpy()
    want = oracle.decode(pool, live, q.f32(), D ** -0.5)
    check_close(got, want, f"decode of {len(live)} live sequences")
    c.close()


INDEPENDENCE = [
    get("tiny_b"),
    scaled("beam", "beam_s", shape=replace_shape(B16, L=3, Hq=8, Hkv=2), root_len=200,
           n_branches=5, branch_len=37),
    scaled("mcts", "mcts_wide", shape=replace_shape(B16, L=2, Hq=16, Hkv=2), root_len=77, depth=4,
           edge_len=19),
    scaled("agent", "agent_s", shape=replace_shape(configs.AGENT, Hq=12, Hkv=2), root_len=300,
           n_branches=3, branch_len=170),
]


@pytest.mark.parametrize("w", INDEPENDENCE, ids=lambda w: w.name)
def test_branch_output_does_not_depend_on_the_batch(pkv, w):
    """Each branch decoded alone and inside its batch: both meet the oracle
    bar against the same oracle row, they agree with each other to fp32
    rounding (the batch only changes how the shared blocks are cut into
    chunks), and a branch decoded alone twice gives identical bits."""
    note(f"independence {w.name}")
    inp = generate(w)
    c, h = build_library(pkv, w, inp)
    pool = build_oracle(w, inp)
    seqs = [h[s] for s in w.query_sids]
    q = inp.q.f32()
    qd = to_device(inp.q)
    batch = c.decode(seqs, qd, scale=w.softmax_scale).cpu().numpy()
    want = oracle.decode(pool, w.query_sids, q, w.softmax_scale)
    check_close(batch, want, f"{w.name} batch")
    worst = 0.0
    for b, sid in enumerate(w.query_sids):
        qb = qd[:, b:b + 1].contiguous()
        alone = c.decode([h[sid]], qb, scale=w.softmax_scale).cpu().numpy()
        again = c.decode([h[sid]], qb, scale=w.softmax_scale).cpu().numpy()
        assert np.array_equal(alone.view(np.uint32), again.view(np.uint32)), sid
        check_close(alone[:, 0], want[:, b], f"{w.name} branch {b} alone")
        worst = max(worst, errors(alone[:, 0], batch[:, b])[0])
    note(f"{w.name}: alone vs batch max |diff| {worst:.3e}")
    assert worst <= 1e-4
    c.close()


@pytest.mark.gpu
def test_stream_read_measuring_aid():
    """pkv_stream_read reads a whole buffer (ordinary and non-temporal loads)
    and leaves it unchanged; the bench's read ceiling comes from it."""
    import torch
    from paged_kv_cache_amd import binding
    a = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    for nt in (True, False):
        binding.pkv_stream_read(a, sink, streaming=nt)
    torch.cuda.synchronize()
    assert torch.equal(a, torch.arange(1 << 20, dtype=torch.int32, device="cuda"))
