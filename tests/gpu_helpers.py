"""GPU-test helpers: build a workload's tree through libpkv on the device and
read the arenas back. No attention or table arithmetic here."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle.pool import OraclePool, run_trace
from workloads import Inputs, Workload

from helpers import kv_for_op


def to_device(t) -> torch.Tensor:
    """A generated Tensor (workloads.gen) as a device tensor of its storage type."""
    if t.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(t.raw)).cuda()
    return torch.from_numpy(np.ascontiguousarray(t.raw).view(np.int16)).cuda().view(torch.bfloat16)


def build_library(pkv, w: Workload, inp: Inputs, alloc_order=None, extra_blocks: int = 8,
                  free_ops: bool = True):
    sh = w.shape
    nb = w.num_blocks_bound() + extra_blocks
    if alloc_order is not None:
        alloc_order = list(alloc_order)[:nb] if len(alloc_order) >= nb else None
    c = pkv.PagedKVCache(nb, sh.BS, sh.L, sh.Hkv, sh.Hq, sh.D, dtype=sh.dtype, device="cuda",
                         alloc_order=alloc_order)
    kv = {i: (k, v) for i, _sid, k, v in inp.appends}
    h = {}
    for i, op in enumerate(w.ops):
        if op.kind == "create":
            h[op.sid] = c.create()
        elif op.kind == "fork":
            h[op.sid] = c.fork(h[op.parent])
        elif op.kind == "append":
            k, v = kv[i]
            c.append([h[op.sid]], [op.n], to_device(k), to_device(v))
        elif op.kind == "free" and free_ops:
            c.free(h.pop(op.sid))
    torch.cuda.synchronize()
    return c, h


def build_oracle(w: Workload, inp: Inputs, free_ops: bool = True) -> OraclePool:
    pool = OraclePool(w.num_blocks_bound() + 8, w.shape.BS)
    if free_ops:
        run_trace(pool, w.ops, kv_for_op(inp))
    else:
        run_trace(pool, [op for op in w.ops if op.kind != "free"], kv_for_op(inp))
    return pool


def arena_bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage bits of an arena on the host (uint16 for bf16, uint32 for f32)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint32)


def gather(c, k_bits: np.ndarray, v_bits: np.ndarray, seq):
    """The sequence's K and V ([L][len][Hkv][D], raw bits) read from the
    arenas through the library's block table."""
    table = np.array(c.table(seq), dtype=np.int64)
    n = c.length(seq)
    L, _, Hkv, BS, D = k_bits.shape
    K = k_bits[:, table].transpose(0, 1, 3, 2, 4).reshape(L, -1, Hkv, D)[:, :n]
    V = v_bits[:, table].transpose(0, 1, 4, 2, 3).reshape(L, -1, Hkv, D)[:, :n]
    return K, V


def raw_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Bits of oracle-materialised float32 values in the storage type."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.view(np.uint32)
    u = x.view(np.uint32)
    assert not np.any(u & 0xFFFF), "value is not a bf16"
    return (u >> 16).astype(np.uint16)


def errors(got: np.ndarray, want: np.ndarray):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    max_abs = float(np.max(np.abs(got - want))) if got.size else 0.0
    rel_l2 = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    return max_abs, rel_l2
