"""DFlash KV-injection attention for MI355X (gfx950).

The layer runs in hand-written HIP kernels behind the C ABI of
include/dflash.h (libdflash.so, built in-tree by `build.py`).  This package
holds that library's sources (csrc/), the ctypes binding (_lib) and the draft
round driver (draft_round), which only sequences ABI calls.

The binding's names are re-exported lazily: importing the package (and so
`block_diffusion_draft_fc_amd.build`) loads no library, so the build runs on a
checkout where libdflash.so is missing or out of date.  The first use of any
of them loads the library and fails loudly if it is missing.
"""
_EXPORTS = (
    "Cache", "DFlashError", "Layer", "LIB_PATH", "dflash_cache_append", "dflash_cache_crop",
    "dflash_ctx_project", "dflash_ctx_project_ws_bytes", "dflash_kv_inject_attn",
    "dflash_kv_inject_attn_ws_bytes", "dtype_code", "strerror",
)
__all__ = list(_EXPORTS)


def __getattr__(name):
    if name in _EXPORTS:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
