"""Agents resuming from the prompt cache, on the device, against the oracle.

Four agents share a system prompt; each turn an agent resumes from the
longest cached prefix of its conversation, appends only the tokens the
cache does not hold, and is snapshotted at the turn boundary. Tables,
counts and K/V bits are bit-exact; decode over the agents meets the decode
bar (max |error| <= 2e-3, relative L2 <= 1e-2 against float64).
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads.gen import Tensor, bf16_round  # noqa: E402

from gpu_helpers import arena_bits, errors, gather, raw_bits, to_device  # noqa: E402

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class TokenKV:
    """K/V of a token as a fixed function of (position, token id), so that a
    prompt recomputed after a resume holds the same values as before."""

    def __init__(self, L, Hkv, D, seed=0):
        self.shape = (L, Hkv, D)
        self.seed = seed

    def __call__(self, ids, start):
        L, Hkv, D = self.shape
        k = np.empty((L, len(ids), Hkv, D), np.float32)
        v = np.empty_like(k)
        for j, t in enumerate(ids):
            rng = np.random.default_rng([self.seed, start + j, int(t)])
            k[:, j] = rng.standard_normal((L, Hkv, D), dtype=np.float32)
            v[:, j] = rng.standard_normal((L, Hkv, D), dtype=np.float32)
        return Tensor(bf16_round(k), "bf16"), Tensor(bf16_round(v), "bf16")


@pytest.mark.parametrize("bs,D,sys_len", [(16, 128, 300), (32, 128, 257), (64, 64, 200)])
def test_agents_resume_from_the_cache(pkv, bs, D, sys_len):
    L, Hkv, Hq = 2, 2, 8
    nb = 160
    note(f"prompt cache agents bs={bs} D={D} system={sys_len}")
    rng = np.random.default_rng(bs + D)
    kvf = TokenKV(L, Hkv, D)
    c = pkv.PagedKVCache(nb, bs, L, Hkv, Hq, D, dtype="bf16", device="cuda")
    pool = oracle.OraclePool(nb, bs)
    system = [int(t) for t in rng.integers(0, 1000, size=sys_len)]
    convs = [list(system) for _ in range(4)]
    live = {}           # agent -> (oracle sid, library handle)
    computed = full = 0
    for turn in range(3):
        for a in range(4):
            convs[a] += [int(t) for t in rng.integers(0, 1000, size=int(rng.integers(5, 40)))]
            if a in live:                      # a conversation that lost its slot resumes
                sid, hd = live.pop(a)
                pool.free(sid)
                c.free(hd)
            sid, m = pool.cache_match(convs[a])
            hd, m2 = c.cache_match(convs[a])
            assert m == m2
            new = convs[a][m:]
            k, v = kvf(new, m)
            pool.append(sid, k.f32(), v.f32())
            c.append([hd], [len(new)], to_device(k), to_device(v))
            computed += len(new)
            full += len(convs[a])
            # the reply, then the snapshot at the turn boundary
            reply = [int(t) for t in rng.integers(0, 1000, size=int(rng.integers(1, 30)))]
            k, v = kvf(reply, len(convs[a]))
            pool.append(sid, k.f32(), v.f32())
            c.append([hd], [len(reply)], to_device(k), to_device(v))
            convs[a] += reply
            assert pool.cache_insert(sid, convs[a]) == c.cache_insert(hd, convs[a])
            live[a] = (sid, hd)
        torch.cuda.synchronize()
        kb, vb = arena_bits(c.k_arena), arena_bits(c.v_arena)
        for a, (sid, hd) in live.items():
            assert c.table(hd) == pool.table(sid), (turn, a)
            K, V = gather(c, kb, vb, hd)
            Ko, Vo = pool.kv(sid)
            assert np.array_equal(K, raw_bits(Ko, "bf16")) and np.array_equal(V, raw_bits(Vo, "bf16"))
            # resumed equals computed in full
            kf, vf = kvf(convs[a], 0)
            assert np.array_equal(Ko, kf.f32()) and np.array_equal(Vo, vf.f32())
        for b in range(nb):
            assert c.refcount(b) == pool.refcount(b)
        assert c.cache_info() == (len(pool.entries), pool.evictable())
    note(f"  prompt tokens computed {computed} of {full} ({100 * (1 - computed / full):.0f}% saved)")
    assert computed < full
    order = sorted(live)
    sids = [live[a][0] for a in order]
    hds = [live[a][1] for a in order]
    q = Tensor(bf16_round(rng.standard_normal((L, 4, Hq, D), dtype=np.float32)), "bf16")
    got = c.decode(hds, to_device(q), scale=D ** -0.5)
    torch.cuda.synchronize()
    want = oracle.decode(pool, sids, q.f32(), D ** -0.5)
    ma, rl = errors(got.cpu().numpy(), want)
    note(f"  decode after resume: max_abs={ma:.3e} rel_l2={rl:.3e}")
    assert ma <= 2e-3 and rl <= 1e-2
    info = c.plan_info(hds)
    assert info["unique_tokens"] < sum(len(x) for x in convs)   # the system prompt is read once
    c.close()
