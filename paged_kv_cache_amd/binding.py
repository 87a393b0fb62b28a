"""Thin Python binding over libpkv's C ABI (include/pkv.h).

The functions keep the C names and only marshal arguments: torch tensors are
passed as device pointers, streams as HIP stream handles (default: torch's
current stream). Every step of the computation runs in the library.
``PagedKVCache`` is a small convenience owner of a pool, its two arenas and
an attention workspace, all allocated through torch.
"""

from __future__ import annotations

import ctypes
from ctypes import byref, c_int32, c_int64, c_size_t, c_void_p
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import _lib
from ._lib import PKV_BF16, PKV_F32, PkvCowOp, PkvPlanInfo, PkvPoolDesc, PkvSeq, PkvStats, check, lib

try:
    import torch
except ImportError:  # pragma: no cover - torch is part of the toolchain
    torch = None


def _dev_ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    if stream is None:
        if torch is None or not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _seq_array(seqs: Sequence[PkvSeq]):
    arr = (PkvSeq * len(seqs))()
    for i, s in enumerate(seqs):
        arr[i] = s
    return arr


# ------------------------------------------------------------- C names

def pkv_pool_create(num_blocks: int, block_size: int, num_layers: int, num_kv_heads: int,
                    num_q_heads: int, head_dim: int, kv_dtype: int,
                    alloc_order: Optional[Sequence[int]] = None, k_arena=None, v_arena=None):
    d = PkvPoolDesc(num_blocks, block_size, num_layers, num_kv_heads, num_q_heads, head_dim, kv_dtype)
    keep = None
    if alloc_order is not None:
        keep = (c_int32 * num_blocks)(*[int(x) for x in alloc_order])
        d.alloc_order = ctypes.cast(keep, ctypes.POINTER(c_int32))
    d.k_arena = _dev_ptr(k_arena)
    d.v_arena = _dev_ptr(v_arena)
    h = c_void_p()
    check(lib.pkv_pool_create(byref(d), byref(h)))
    return h


def pkv_pool_destroy(pool) -> None:
    check(lib.pkv_pool_destroy(pool))


def pkv_arena_bytes(num_blocks, block_size, num_layers, num_kv_heads, num_q_heads, head_dim,
                    kv_dtype) -> int:
    d = PkvPoolDesc(num_blocks, block_size, num_layers, num_kv_heads, num_q_heads, head_dim, kv_dtype)
    out = c_size_t()
    check(lib.pkv_arena_bytes(byref(d), byref(out)))
    return out.value


def pkv_block_alloc(pool) -> int:
    b = c_int32()
    check(lib.pkv_block_alloc(pool, byref(b)))
    return b.value


def pkv_block_release(pool, block: int) -> None:
    check(lib.pkv_block_release(pool, block))


def pkv_seq_create(pool) -> PkvSeq:
    s = PkvSeq()
    check(lib.pkv_seq_create(pool, byref(s)))
    return s


def pkv_seq_fork(pool, parent: PkvSeq) -> PkvSeq:
    c = PkvSeq()
    check(lib.pkv_seq_fork(pool, parent, byref(c)))
    return c


def pkv_seq_free(pool, seq: PkvSeq) -> None:
    check(lib.pkv_seq_free(pool, seq))


def pkv_seq_fork_many(pool, parents: Sequence[PkvSeq]) -> List[PkvSeq]:
    kids = (PkvSeq * max(len(parents), 1))()
    check(lib.pkv_seq_fork_many(pool, _seq_array(parents), len(parents), kids))
    return list(kids[:len(parents)])


def pkv_seq_free_many(pool, seqs: Sequence[PkvSeq]) -> None:
    check(lib.pkv_seq_free_many(pool, _seq_array(seqs), len(seqs)))


def pkv_seq_append_plan(pool, seq: PkvSeq, n: int) -> Tuple[List[int], List[Tuple[int, int, int]]]:
    slots = (c_int64 * max(n, 1))()
    cow = PkvCowOp()
    ncow = c_int32()
    check(lib.pkv_seq_append_plan(pool, seq, n, slots, byref(cow), byref(ncow)))
    cows = [(cow.src, cow.dst, cow.n_valid)] if ncow.value else []
    return list(slots[:n]), cows


def pkv_cow_copy(pool, ops: Sequence[Tuple[int, int, int]], stream=None) -> None:
    arr = (PkvCowOp * max(len(ops), 1))(*[PkvCowOp(*o) for o in ops])
    check(lib.pkv_cow_copy(pool, arr, len(ops), _stream(stream)))


def pkv_write_kv(pool, slots: Sequence[int], k_new, v_new, stream=None) -> None:
    arr = (c_int64 * max(len(slots), 1))(*[int(s) for s in slots])
    check(lib.pkv_write_kv(pool, arr, len(slots), _dev_ptr(k_new), _dev_ptr(v_new), _stream(stream)))


def pkv_append_kv_batch(pool, seqs: Sequence[PkvSeq], counts: Sequence[int], k_new, v_new,
                        stream=None) -> None:
    sa = _seq_array(seqs)
    ca = (c_int32 * max(len(counts), 1))(*[int(c) for c in counts])
    check(lib.pkv_append_kv_batch(pool, sa, ca, len(seqs), _dev_ptr(k_new), _dev_ptr(v_new),
                                  _stream(stream)))


def pkv_seq_append_kv(pool, seq: PkvSeq, n: int, k_new, v_new, stream=None) -> None:
    check(lib.pkv_seq_append_kv(pool, seq, n, _dev_ptr(k_new), _dev_ptr(v_new), _stream(stream)))


def pkv_seq_info(pool, seq: PkvSeq) -> Tuple[int, int]:
    ln, nb = c_int32(), c_int32()
    check(lib.pkv_seq_info(pool, seq, byref(ln), byref(nb)))
    return ln.value, nb.value


def pkv_seq_blocks(pool, seq: PkvSeq) -> List[int]:
    _, nb = pkv_seq_info(pool, seq)
    out = (c_int32 * max(nb, 1))()
    check(lib.pkv_seq_blocks(pool, seq, out, nb))
    return list(out[:nb])


def pkv_block_refcount(pool, block: int) -> int:
    rc = c_int32()
    check(lib.pkv_block_refcount(pool, block, byref(rc)))
    return rc.value


def pkv_block_refcounts(pool, n: int) -> List[int]:
    out = (c_int32 * max(n, 1))()
    check(lib.pkv_block_refcounts(pool, out, n))
    return list(out[:n])


def pkv_pool_stats(pool) -> dict:
    st = PkvStats()
    check(lib.pkv_pool_stats(pool, byref(st)))
    return {"num_blocks": st.num_blocks, "free_blocks": st.free_blocks, "live_seqs": st.live_seqs,
            "total_refs": st.total_refs, "table_ids_copied": st.table_ids_copied}


def pkv_pool_set_option(pool, key: str, value: int) -> None:
    check(lib.pkv_pool_set_option(pool, key.encode(), int(value)))


def pkv_timing_read(pool, kernel: str) -> Tuple[float, int]:
    ms = ctypes.c_double()
    n = c_int64()
    check(lib.pkv_timing_read(pool, kernel.encode(), byref(ms), byref(n)))
    return ms.value, n.value


def pkv_stream_read(src, sink, streaming: bool = True, stream=None) -> None:
    """Reads the whole of the contiguous device tensor src once (a measuring
    aid: the practical HBM read rate); sink: a device tensor of >= 4096
    bytes."""
    check(lib.pkv_stream_read(_dev_ptr(src), src.numel() * src.element_size(), 1 if streaming else 0,
                              _dev_ptr(sink), _stream(stream)))


def pkv_decode_plan_info(pool, seqs: Sequence[PkvSeq], n_layers: int) -> dict:
    info = PkvPlanInfo()
    check(lib.pkv_decode_plan_info(pool, _seq_array(seqs), len(seqs), n_layers, byref(info)))
    return {k: getattr(info, k) for k, _ in PkvPlanInfo._fields_}


def pkv_decode_workspace_size(pool, seqs: Sequence[PkvSeq], n_layers: int) -> int:
    out = c_size_t()
    check(lib.pkv_decode_workspace_size(pool, _seq_array(seqs), len(seqs), n_layers, byref(out)))
    return out.value


def pkv_decode_attn(pool, seqs: Sequence[PkvSeq], layer0: int, n_layers: int, q, out, scale: float,
                    ws, stream=None) -> None:
    check(lib.pkv_decode_attn(pool, _seq_array(seqs), len(seqs), layer0, n_layers, _dev_ptr(q),
                              _dev_ptr(out), float(scale), _dev_ptr(ws), ws.numel() * ws.element_size(),
                              _stream(stream)))


def pkv_decode_attn_noalloc(pool, seqs: Sequence[PkvSeq], layer0: int, n_layers: int, q, out,
                            scale: float, stream=None) -> None:
    check(lib.pkv_decode_attn_noalloc(pool, _seq_array(seqs), len(seqs), layer0, n_layers,
                                      _dev_ptr(q), _dev_ptr(out), float(scale), _stream(stream)))


def pkv_verify_workspace_size(pool, reqs: Sequence[PkvSeq], n_nodes: int) -> int:
    out = c_size_t()
    check(lib.pkv_verify_workspace_size(pool, _seq_array(reqs), len(reqs), n_nodes, byref(out)))
    return out.value


def pkv_tree_verify_attn(pool, reqs: Sequence[PkvSeq], parents, layer: int, q, out, scale: float,
                         ws, stream=None) -> None:
    par = np.ascontiguousarray(np.asarray(parents, dtype=np.int32))
    n_nodes = par.shape[-1]
    pa = par.ctypes.data_as(ctypes.POINTER(c_int32))
    check(lib.pkv_tree_verify_attn(pool, _seq_array(reqs), len(reqs), pa, n_nodes, layer,
                                   _dev_ptr(q), _dev_ptr(out), float(scale), _dev_ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)))


def pkv_seq_truncate(pool, seq: PkvSeq, new_len: int) -> None:
    check(lib.pkv_seq_truncate(pool, seq, int(new_len)))


def pkv_tree_commit_workspace_size(pool, n_accepted: int) -> int:
    out = c_size_t()
    check(lib.pkv_tree_commit_workspace_size(pool, int(n_accepted), byref(out)))
    return out.value


def pkv_tree_commit(pool, seq: PkvSeq, parents, accepted, ws, stream=None) -> None:
    par = np.ascontiguousarray(np.asarray(parents, dtype=np.int32).reshape(-1))
    acc = np.ascontiguousarray(np.asarray(accepted, dtype=np.int32).reshape(-1))
    acc_buf = acc if acc.size else np.zeros(1, dtype=np.int32)
    check(lib.pkv_tree_commit(pool, seq, par.size, par.ctypes.data_as(ctypes.POINTER(c_int32)),
                              acc_buf.ctypes.data_as(ctypes.POINTER(c_int32)), acc.size,
                              _dev_ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                              _stream(stream)))


def pkv_tree_commit_batch(pool, seqs: Sequence[PkvSeq], parents, accepted: Sequence[Sequence[int]],
                          ws, stream=None) -> None:
    par = np.ascontiguousarray(np.asarray(parents, dtype=np.int32))
    n_req, n_nodes = par.shape
    acc = np.full((n_req, n_nodes), -1, dtype=np.int32)
    na = np.zeros(n_req, dtype=np.int32)
    for r, path in enumerate(accepted):
        path = list(path)
        if len(path) > n_nodes:
            raise ValueError("a path is longer than the tree")
        acc[r, :len(path)] = path
        na[r] = len(path)
    check(lib.pkv_tree_commit_batch(pool, _seq_array(seqs), n_req, n_nodes,
                                    par.ctypes.data_as(ctypes.POINTER(c_int32)),
                                    acc.ctypes.data_as(ctypes.POINTER(c_int32)),
                                    na.ctypes.data_as(ctypes.POINTER(c_int32)),
                                    _dev_ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(stream)))


def _tokens(tokens):
    t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
    buf = t if t.size else np.zeros(1, dtype=np.int32)
    return t.size, buf, buf.ctypes.data_as(ctypes.POINTER(c_int32))


def pkv_prefix_insert(pool, seq: PkvSeq, tokens) -> int:
    n, _buf, ptr = _tokens(tokens)
    added = c_int32()
    check(lib.pkv_prefix_insert(pool, seq, ptr, n, byref(added)))
    return added.value


def pkv_prefix_match(pool, tokens) -> Tuple[PkvSeq, int]:
    n, _buf, ptr = _tokens(tokens)
    out, matched = PkvSeq(), c_int32()
    check(lib.pkv_prefix_match(pool, ptr, n, byref(out), byref(matched)))
    return out, matched.value


def pkv_prefix_clear(pool) -> None:
    check(lib.pkv_prefix_clear(pool))


def pkv_prefix_info(pool) -> Tuple[int, int]:
    entries, evictable = c_int32(), c_int32()
    check(lib.pkv_prefix_info(pool, byref(entries), byref(evictable)))
    return entries.value, evictable.value


def pkv_last_error() -> str:
    return lib.pkv_last_error().decode(errors="replace")


def pkv_version() -> str:
    return lib.pkv_version().decode()


# ------------------------------------------------------- convenience owner

class PagedKVCache:
    """A pool plus its K/V arenas and a reusable attention workspace.

    K arena: [L][NB][Hkv][BS][D]; V arena: [L][NB][Hkv][D][BS] (see pkv.h).
    With ``device=None`` no arenas are allocated (host-side table work only).
    """

    def __init__(self, num_blocks: int, block_size: int, num_layers: int, num_kv_heads: int,
                 num_q_heads: int, head_dim: int, dtype: str = "bf16", device="cuda",
                 alloc_order: Optional[Sequence[int]] = None):
        self.NB, self.BS, self.L = num_blocks, block_size, num_layers
        self.Hkv, self.Hq, self.D = num_kv_heads, num_q_heads, head_dim
        self.dtype = dtype
        self.kv_dtype = PKV_BF16 if dtype == "bf16" else PKV_F32
        self.k_arena = self.v_arena = None
        if device is not None:
            tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
            self.k_arena = torch.empty((num_layers, num_blocks, num_kv_heads, block_size, head_dim),
                                       dtype=tdt, device=device)
            self.v_arena = torch.empty((num_layers, num_blocks, num_kv_heads, head_dim, block_size),
                                       dtype=tdt, device=device)
        self.handle = pkv_pool_create(num_blocks, block_size, num_layers, num_kv_heads, num_q_heads,
                                      head_dim, self.kv_dtype, alloc_order, self.k_arena, self.v_arena)
        self.ws = None

    def close(self) -> None:
        if self.handle is not None:
            pkv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # table verbs
    def create(self) -> PkvSeq:
        return pkv_seq_create(self.handle)

    def fork(self, parent: PkvSeq) -> PkvSeq:
        return pkv_seq_fork(self.handle, parent)

    def free(self, seq: PkvSeq) -> None:
        pkv_seq_free(self.handle, seq)

    def fork_many(self, parents: Sequence[PkvSeq]) -> List[PkvSeq]:
        return pkv_seq_fork_many(self.handle, parents)

    def free_many(self, seqs: Sequence[PkvSeq]) -> None:
        pkv_seq_free_many(self.handle, seqs)

    def plan(self, seq: PkvSeq, n: int):
        return pkv_seq_append_plan(self.handle, seq, n)

    def table(self, seq: PkvSeq) -> List[int]:
        return pkv_seq_blocks(self.handle, seq)

    def length(self, seq: PkvSeq) -> int:
        return pkv_seq_info(self.handle, seq)[0]

    def truncate(self, seq: PkvSeq, new_len: int) -> None:
        pkv_seq_truncate(self.handle, seq, new_len)

    # prompt cache
    def cache_insert(self, seq: PkvSeq, tokens) -> int:
        return pkv_prefix_insert(self.handle, seq, tokens)

    def cache_match(self, tokens) -> Tuple[PkvSeq, int]:
        return pkv_prefix_match(self.handle, tokens)

    def cache_clear(self) -> None:
        pkv_prefix_clear(self.handle)

    def cache_info(self) -> Tuple[int, int]:
        return pkv_prefix_info(self.handle)

    def refcount(self, block: int) -> int:
        return pkv_block_refcount(self.handle, block)

    def refcounts(self) -> List[int]:
        return pkv_block_refcounts(self.handle, self.NB)

    def stats(self) -> dict:
        return pkv_pool_stats(self.handle)

    def timing_read(self, kernel: str) -> Tuple[float, int]:
        return pkv_timing_read(self.handle, kernel)

    def plan_info(self, seqs: Sequence[PkvSeq], n_layers: Optional[int] = None) -> dict:
        return pkv_decode_plan_info(self.handle, seqs, self.L if n_layers is None else n_layers)

    def set_option(self, key: str, value: int) -> None:
        pkv_pool_set_option(self.handle, key, value)

    # attention
    def _check_q(self, q, shape):
        want = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        if tuple(q.shape) != tuple(shape) or q.dtype != want or not q.is_contiguous():
            raise ValueError(f"q must be a contiguous {want} tensor of shape {shape}")

    def _check_out(self, out, shape):
        if tuple(out.shape) != tuple(shape) or out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous float32 tensor of shape {shape}")

    def append(self, seqs: Sequence[PkvSeq], counts: Sequence[int], k_new, v_new, stream=None) -> None:
        want = (self.L, int(sum(counts)), self.Hkv, self.D)
        for t in (k_new, v_new):
            if tuple(t.shape) != want or not t.is_contiguous():
                raise ValueError(f"new K/V must be contiguous tensors of shape {want}")
        pkv_append_kv_batch(self.handle, seqs, counts, k_new, v_new, stream)

    def _workspace(self, nbytes: int):
        if self.ws is None or self.ws.numel() < nbytes:
            self.ws = torch.empty(max(nbytes, 1 << 16), dtype=torch.uint8, device=self.k_arena.device)
        return self.ws

    def decode(self, seqs: Sequence[PkvSeq], q, layer0: int = 0, n_layers: Optional[int] = None,
               scale: Optional[float] = None, out=None, stream=None):
        n_layers = self.L - layer0 if n_layers is None else n_layers
        scale = self.D ** -0.5 if scale is None else scale
        self._check_q(q, (n_layers, len(seqs), self.Hq, self.D))
        ws = self._workspace(pkv_decode_workspace_size(self.handle, seqs, n_layers))
        if out is None:
            out = torch.empty((n_layers, len(seqs), self.Hq, self.D), dtype=torch.float32,
                              device=self.k_arena.device)
        self._check_out(out, (n_layers, len(seqs), self.Hq, self.D))
        pkv_decode_attn(self.handle, seqs, layer0, n_layers, q, out, scale, ws, stream)
        return out

    def verify(self, reqs: Sequence[PkvSeq], parents, q, layer: int = 0,
               scale: Optional[float] = None, out=None, stream=None):
        par = np.asarray(parents, dtype=np.int32)
        scale = self.D ** -0.5 if scale is None else scale
        if par.shape != (len(reqs), par.shape[-1]):
            raise ValueError("parents must be [n_req][n_nodes]")
        self._check_q(q, (len(reqs), par.shape[-1], self.Hq, self.D))
        ws = self._workspace(pkv_verify_workspace_size(self.handle, reqs, par.shape[-1]))
        if out is None:
            out = torch.empty((len(reqs), par.shape[-1], self.Hq, self.D), dtype=torch.float32,
                              device=self.k_arena.device)
        self._check_out(out, (len(reqs), par.shape[-1], self.Hq, self.D))
        pkv_tree_verify_attn(self.handle, reqs, par, layer, q, out, scale, ws, stream)
        return out

    def commit(self, seq: PkvSeq, parents, accepted, stream=None) -> None:
        """Keeps the accepted root-to-node path of the draft tree that ends seq."""
        ws = self._workspace(pkv_tree_commit_workspace_size(self.handle, len(accepted)))
        pkv_tree_commit(self.handle, seq, parents, accepted, ws, stream)

    def commit_batch(self, seqs: Sequence[PkvSeq], parents, accepted, stream=None) -> None:
        """commit for several requests of one verify step in one call."""
        if len(accepted) != len(seqs):
            raise ValueError("one accepted path per request")
        total = sum(len(a) for a in accepted)
        ws = self._workspace(pkv_tree_commit_workspace_size(self.handle, total))
        pkv_tree_commit_batch(self.handle, seqs, parents, accepted, ws, stream)
