"""paged_kv_cache_amd: a copy-on-write paged KV cache for tree-structured
decoding on AMD MI355X (gfx950).

The work happens in ``libpkv.so`` (HIP kernels plus a C++ host pool, C ABI
in ``include/pkv.h``); this package only loads it and marshals arguments.
Importing it without the built library raises ImportError.
"""

from .binding import *  # noqa: F401,F403
from .binding import PagedKVCache  # noqa: F401
from ._lib import (  # noqa: F401
    LIB_PATH,
    OOM,
    PKV_BF16,
    PKV_E_HIP,
    PKV_E_INVALID,
    PKV_E_OOM,
    PKV_E_UNSUPPORTED,
    PKV_E_WORKSPACE,
    PKV_F32,
    PkvError,
    PkvSeq,
)
