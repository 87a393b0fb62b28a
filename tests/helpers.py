"""Shared test helpers. Nothing here computes attention or block tables."""

from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

from workloads import Inputs, Workload


def assemble_sequences(w: Workload, inp: Inputs) -> Dict[int, Tuple[np.ndarray, np.ndarray]]:
    """Each live sequence's logical K/V ([L][len][Hkv][D] float32), assembled
    straight from the trace: a forked sequence starts as its parent's tokens,
    an append adds its tokens at the end. Independent of any block pool."""
    kv_of_op = {i: (k.f32(), v.f32()) for i, _sid, k, v in inp.appends}
    seqs: Dict[int, list] = {}
    for i, op in enumerate(w.ops):
        if op.kind == "create":
            seqs[op.sid] = []
        elif op.kind == "fork":
            seqs[op.sid] = list(seqs[op.parent])
        elif op.kind == "append":
            seqs[op.sid] = seqs[op.sid] + [kv_of_op[i]]
        elif op.kind == "free":
            del seqs[op.sid]
    return {s: (np.concatenate([c[0] for c in chunks], axis=1),
                np.concatenate([c[1] for c in chunks], axis=1))
            for s, chunks in seqs.items() if chunks}


def kv_for_op(inp: Inputs):
    """Map op index -> (K, V) float32 arrays, for oracle.pool.run_trace."""
    table = {i: (k, v) for i, _sid, k, v in inp.appends}

    def get(i):
        k, v = table[i]
        return k.f32(), v.f32()
    return get


def structure_only_kv(i_unused=None, n=0):
    return np.zeros((1, n, 1, 1), np.float32), np.zeros((1, n, 1, 1), np.float32)


def run_structure(pool, w: Workload):
    """Run a trace with empty K/V payloads (shape [1][n][1][1]) -- enough for
    tables and refcounts, cheap for the full-size workloads."""
    for op in w.ops:
        if op.kind == "create":
            pool.create(op.sid)
        elif op.kind == "fork":
            pool.fork(op.parent, op.sid)
        elif op.kind == "append":
            k, v = structure_only_kv(n=op.n)
            pool.append(op.sid, k, v)
        elif op.kind == "free":
            pool.free(op.sid)
