"""Oracle attention: the plain definition, softmax(q K^T * scale) V, in float64.

Test infrastructure (see the package docstring). No blocking, no split of the
sequence, no online rescaling: each output is one softmax over the whole set
of keys it may see.

Readings used here:

* Grouped-query heads: query head h reads KV head h // G with G = Hq / Hkv
  (contiguous groups).
* A decode query attends to every token its sequence holds, its own token
  included (that token's K/V were appended before the attention call).
* Verify: the last ``N`` tokens of a request are the draft-tree nodes, node j
  at position ``len - N + j``. Node i sees the whole context (positions
  below ``len - N``) and the nodes on its path to the root, itself included
  (Ferrite page, section 04: drafts verified as best-first trees in one pass).
  ``parents[i]`` is -1 for a node hanging off the context, otherwise an
  earlier node.
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from .pool import InvalidError, OraclePool


def _softmax_attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Q [m][D], K [n][D], V [n][D] -> [m][D]; float64 throughout."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    x = (Q @ K.T) * scale
    x = x - x.max(axis=1, keepdims=True)
    p = np.exp(x)
    return (p @ V) / p.sum(axis=1, keepdims=True)


def decode(pool: OraclePool, sids: Sequence[int], q: np.ndarray, scale: float,
           layers: Optional[Sequence[int]] = None) -> np.ndarray:
    """q [L][B][Hq][D] (float), one query per sequence ``sids[b]`` and head.
    Returns [len(layers)][B][Hq][D] float64. ``layers`` defaults to all."""
    L, B, Hq, D = q.shape
    if B != len(sids):
        raise InvalidError("q batch does not match the sequence list")
    layers = list(range(L)) if layers is None else list(layers)
    out = np.empty((len(layers), B, Hq, D), dtype=np.float64)
    for b, s in enumerate(sids):
        for li, l in enumerate(layers):
            K, V = pool.kv(s, layer=l)          # [len][Hkv][D]
            Hkv = K.shape[1]
            if Hq % Hkv:
                raise InvalidError("Hq must be a multiple of Hkv")
            G = Hq // Hkv
            for g in range(Hkv):
                out[li, b, g * G:(g + 1) * G] = _softmax_attend(
                    q[l, b, g * G:(g + 1) * G], K[:, g, :], V[:, g, :], scale)
    return out


def decode_one(pool: OraclePool, sid: int, qvec: np.ndarray, layer: int, head: int,
               num_q_heads: int, scale: float) -> np.ndarray:
    """One output row: sequence ``sid``, layer ``layer``, query head ``head``."""
    K, V = pool.kv(sid, layer=layer)
    G = num_q_heads // K.shape[1]
    g = head // G
    return _softmax_attend(qvec[None, :], K[:, g, :], V[:, g, :], scale)[0]


def ancestors(parents: Sequence[int], i: int) -> List[int]:
    """Node i and every node on its path to the root, in ascending order."""
    out = []
    j = int(i)
    while j != -1:
        if j < 0 or j >= len(parents) or (out and j >= out[-1]):
            raise InvalidError("parents must point to earlier nodes or -1")
        out.append(j)
        j = int(parents[j])
    return sorted(out)


def verify(pool: OraclePool, reqs: Sequence[int], parents: np.ndarray, q: np.ndarray,
           scale: float, layer: int = 0) -> np.ndarray:
    """q [R][N][Hq][D]; parents int [R][N]. Returns [R][N][Hq][D] float64."""
    R, N, Hq, D = q.shape
    out = np.empty((R, N, Hq, D), dtype=np.float64)
    for r, s in enumerate(reqs):
        K, V = pool.kv(s, layer=layer)
        total = K.shape[0]
        c = total - N
        if c < 0:
            raise InvalidError("request shorter than its draft tree")
        Hkv = K.shape[1]
        G = Hq // Hkv
        for i in range(N):
            idx = np.concatenate([np.arange(c), c + np.asarray(ancestors(parents[r], i), dtype=np.int64)])
            for g in range(Hkv):
                out[r, i, g * G:(g + 1) * G] = _softmax_attend(
                    q[r, i, g * G:(g + 1) * G], K[idx, g, :], V[idx, g, :], scale)
    return out
