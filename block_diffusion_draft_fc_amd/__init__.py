"""DFlash KV-injection attention for MI355X (gfx950).

The layer runs in hand-written HIP kernels behind the C ABI of
include/dflash.h (libdflash.so, built in-tree by `build.py`).  This package
holds that library's sources (csrc/), the ctypes binding (_lib) and the draft
round driver (draft_round), which only sequences ABI calls.
"""
from ._lib import (  # noqa: F401
    Cache, DFlashError, Layer, LIB_PATH, dflash_cache_append, dflash_cache_crop,
    dflash_ctx_project, dflash_ctx_project_ws_bytes, dflash_kv_inject_attn,
    dflash_kv_inject_attn_ws_bytes, dtype_code, strerror,
)
