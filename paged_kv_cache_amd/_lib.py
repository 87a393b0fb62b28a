"""ctypes loader for libpkv.so (the C ABI in include/pkv.h).

Marshalling only: structures, argument types and error codes. The library
must have been built (``python -m paged_kv_cache_amd.build``); importing
this module without it raises ImportError -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_uint32, c_void_p

# PKV_LIBRARY names another build of the same library (the sanitizer build
# of the host runtime, ``build.py --sanitize``); by default the in-tree one.
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_OK = 0
PKV_E_INVALID = -1
PKV_E_OOM = -2
PKV_E_HIP = -3
PKV_E_UNSUPPORTED = -4
PKV_E_WORKSPACE = -5
PKV_F32 = 0
PKV_BF16 = 1


class PkvSeq(ctypes.Structure):
    _fields_ = [("index", c_int32), ("generation", c_uint32)]

    def key(self):
        return (self.index, self.generation)

    def __repr__(self):
        return f"PkvSeq({self.index}, gen={self.generation})"


class PkvCowOp(ctypes.Structure):
    _fields_ = [("src", c_int32), ("dst", c_int32), ("n_valid", c_int32)]


class PkvPoolDesc(ctypes.Structure):
    _fields_ = [("num_blocks", c_int32), ("block_size", c_int32), ("num_layers", c_int32),
                ("num_kv_heads", c_int32), ("num_q_heads", c_int32), ("head_dim", c_int32),
                ("kv_dtype", c_int32), ("alloc_order", POINTER(c_int32)),
                ("k_arena", c_void_p), ("v_arena", c_void_p)]


class PkvStats(ctypes.Structure):
    _fields_ = [("num_blocks", c_int32), ("free_blocks", c_int32), ("live_seqs", c_int32),
                ("reserved", c_int32), ("total_refs", c_int64),
                ("table_ids_copied", c_int64)]


class PkvPlanInfo(ctypes.Structure):
    _fields_ = [("n_segments", c_int32), ("n_chunks", c_int32), ("n_items", c_int32),
                ("partial_rows", c_int32), ("unique_tokens", c_int64), ("workspace_bytes", c_int64),
                ("plan_bytes", c_int64), ("wide_tokens", c_int64), ("read_tokens", c_int64),
                ("grouped_items", c_int32), ("reserved", c_int32)]


class PkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"pkv error {code}: {msg}")
        self.code = code


class OOM(PkvError):
    pass


# name -> (restype, argtypes); every call returns an int status unless noted
_PROTOS = {
    "pkv_pool_create": [POINTER(PkvPoolDesc), POINTER(c_void_p)],
    "pkv_pool_destroy": [c_void_p],
    "pkv_block_alloc": [c_void_p, POINTER(c_int32)],
    "pkv_block_release": [c_void_p, c_int32],
    "pkv_seq_create": [c_void_p, POINTER(PkvSeq)],
    "pkv_seq_fork": [c_void_p, PkvSeq, POINTER(PkvSeq)],
    "pkv_seq_free": [c_void_p, PkvSeq],
    "pkv_seq_fork_many": [c_void_p, POINTER(PkvSeq), c_int32, POINTER(PkvSeq)],
    "pkv_seq_free_many": [c_void_p, POINTER(PkvSeq), c_int32],
    "pkv_seq_append_plan": [c_void_p, PkvSeq, c_int32, POINTER(c_int64), POINTER(PkvCowOp),
                            POINTER(c_int32)],
    "pkv_cow_copy": [c_void_p, POINTER(PkvCowOp), c_int32, c_void_p],
    "pkv_write_kv": [c_void_p, POINTER(c_int64), c_int32, c_void_p, c_void_p, c_void_p],
    "pkv_append_kv_batch": [c_void_p, POINTER(PkvSeq), POINTER(c_int32), c_int32, c_void_p,
                            c_void_p, c_void_p],
    "pkv_seq_append_kv": [c_void_p, PkvSeq, c_int32, c_void_p, c_void_p, c_void_p],
    "pkv_seq_info": [c_void_p, PkvSeq, POINTER(c_int32), POINTER(c_int32)],
    "pkv_seq_blocks": [c_void_p, PkvSeq, POINTER(c_int32), c_int32],
    "pkv_block_refcount": [c_void_p, c_int32, POINTER(c_int32)],
    "pkv_block_refcounts": [c_void_p, POINTER(c_int32), c_int32],
    "pkv_pool_stats": [c_void_p, POINTER(PkvStats)],
    "pkv_arena_bytes": [POINTER(PkvPoolDesc), POINTER(c_size_t)],
    "pkv_decode_plan_info": [c_void_p, POINTER(PkvSeq), c_int32, c_int32, POINTER(PkvPlanInfo)],
    "pkv_decode_workspace_size": [c_void_p, POINTER(PkvSeq), c_int32, c_int32, POINTER(c_size_t)],
    "pkv_decode_attn": [c_void_p, POINTER(PkvSeq), c_int32, c_int32, c_int32, c_void_p, c_void_p,
                        c_float, c_void_p, c_size_t, c_void_p],
    "pkv_decode_attn_noalloc": [c_void_p, POINTER(PkvSeq), c_int32, c_int32, c_int32, c_void_p,
                                c_void_p, c_float, c_void_p],
    "pkv_verify_workspace_size": [c_void_p, POINTER(PkvSeq), c_int32, c_int32, POINTER(c_size_t)],
    "pkv_tree_verify_attn": [c_void_p, POINTER(PkvSeq), c_int32, POINTER(c_int32), c_int32, c_int32,
                             c_void_p, c_void_p, c_float, c_void_p, c_size_t, c_void_p],
    "pkv_seq_truncate": [c_void_p, PkvSeq, c_int32],
    "pkv_tree_commit_workspace_size": [c_void_p, c_int32, POINTER(c_size_t)],
    "pkv_tree_commit": [c_void_p, PkvSeq, c_int32, POINTER(c_int32), POINTER(c_int32), c_int32,
                        c_void_p, c_size_t, c_void_p],
    "pkv_tree_commit_batch": [c_void_p, POINTER(PkvSeq), c_int32, c_int32, POINTER(c_int32),
                              POINTER(c_int32), POINTER(c_int32), c_void_p, c_size_t, c_void_p],
    "pkv_prefix_insert": [c_void_p, PkvSeq, POINTER(c_int32), c_int32, POINTER(c_int32)],
    "pkv_prefix_match": [c_void_p, POINTER(c_int32), c_int32, POINTER(PkvSeq), POINTER(c_int32)],
    "pkv_prefix_clear": [c_void_p],
    "pkv_prefix_info": [c_void_p, POINTER(c_int32), POINTER(c_int32)],
    "pkv_pool_set_option": [c_void_p, c_char_p, c_int64],
    "pkv_timing_read": [c_void_p, c_char_p, POINTER(ctypes.c_double), POINTER(c_int64)],
    "pkv_stream_read": [c_void_p, c_int64, c_int32, c_void_p, c_void_p],
}
_STRING_FUNCS = ("pkv_last_error", "pkv_version")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libpkv.so is not built ({LIB_PATH}); run python -m paged_kv_cache_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in _PROTOS.items():
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = args
    for name in _STRING_FUNCS:
        fn = getattr(lib, name)
        fn.restype = c_char_p
        fn.argtypes = []
    return lib


lib = _load()


def check(rc: int) -> None:
    if rc != PKV_OK:
        msg = lib.pkv_last_error().decode(errors="replace")
        raise (OOM if rc == PKV_E_OOM else PkvError)(rc, msg)


def declared_symbols():
    return list(_PROTOS) + list(_STRING_FUNCS)
