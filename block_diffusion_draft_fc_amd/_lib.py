"""ctypes binding of libdflash.so (include/dflash.h).

Argument marshalling only: torch tensors become device pointers, the current
HIP stream becomes the stream argument, and negative status codes become
DFlashError.  Every step of the layer runs in the library's HIP kernels.  If
the library has not been built, importing the binding raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdflash.so")

DFLASH_OK = 0
ERR_ARG, ERR_SHAPE, ERR_DTYPE, ERR_RANGE, ERR_CAPACITY, ERR_HIP, ERR_WORKSPACE = -1, -2, -3, -4, -5, -6, -7
DFLASH_F32, DFLASH_BF16, DFLASH_FP8_E4M3 = 0, 1, 2


class DFlashError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {strerror(code)} ({code})")
        self.code = code


class LayerDesc(C.Structure):
    _fields_ = [("d", C.c_int32), ("n_h", C.c_int32), ("n_kv", C.c_int32), ("d_h", C.c_int32),
                ("eps", C.c_float), ("rope_theta", C.c_double), ("window", C.c_int32),
                ("dtype", C.c_int32), ("residual", C.c_int32), ("w_qkv", C.c_void_p), ("w_o", C.c_void_p),
                ("gamma_q", C.c_void_p), ("gamma_k", C.c_void_p)]


class CacheDesc(C.Structure):
    _fields_ = [("n_seqs", C.c_int32), ("n_kv", C.c_int32), ("d_h", C.c_int32), ("dtype", C.c_int32),
                ("page_size", C.c_int32), ("max_pages_per_seq", C.c_int32), ("ring", C.c_int32),
                ("capacity", C.c_int64),
                ("k_pool", C.c_void_p), ("v_pool", C.c_void_p), ("block_table", C.c_void_p),
                ("k_scale", C.c_float), ("v_scale", C.c_float)]


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m block_diffusion_draft_fc_amd.build` (there is no CPU fallback)")
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    p32 = C.POINTER(C.c_int32)
    sig = {
        "dflash_strerror": (C.c_char_p, [C.c_int]),
        "dflash_cache_init": (C.c_int, [C.POINTER(vp), C.POINTER(CacheDesc)]),
        "dflash_cache_destroy": (C.c_int, [vp]),
        "dflash_cache_lengths": (C.c_int, [vp, p32]),
        "dflash_cache_block_table": (C.c_int, [vp, p32]),
        "dflash_cache_free_pages": (i64, [vp]),
        "dflash_ctx_project_ws_bytes": (sz, [i64, i64, i64, i32]),
        "dflash_ctx_project": (C.c_int, [vp, i64, i64, vp, vp, i64, C.c_float, i32, vp, vp, sz, vp]),
        "dflash_cache_append": (C.c_int, [vp, p32, vp, vp, vp]),
        "dflash_cache_crop": (C.c_int, [vp, p32, vp]),
        "dflash_kv_inject_attn_ws_bytes": (sz, [C.POINTER(LayerDesc), vp, i64, i32]),
        "dflash_kv_inject_attn": (C.c_int, [C.POINTER(LayerDesc), vp, vp, p32, vp, i32, vp, vp, sz, vp]),
        "dflash_kv_inject_attn_noalloc": (C.c_int, [C.POINTER(LayerDesc), vp, vp, p32, vp, i32, vp, vp]),
        "dflash_cache_device_begin": (C.c_int, [vp, vp, vp]),
        "dflash_kv_inject_attn_dev_ws_bytes": (sz, [C.POINTER(LayerDesc), vp, i32, i32]),
        "dflash_kv_inject_attn_dev": (C.c_int, [C.POINTER(LayerDesc), vp, vp, i32, vp, vp, i32, vp, vp, sz, vp]),
        "dflash_cache_crop_tail_dev": (C.c_int, [vp, i32, vp]),
        "dflash_cache_device_end": (C.c_int, [vp, vp]),
        "dflash_cache_device_reset": (C.c_int, [vp, p32, vp]),
        "dflash_draft_head_ws_bytes": (sz, [i64, i32, i64, i64, i32]),
        "dflash_draft_head": (C.c_int, [vp, i64, i32, i64, vp, C.c_float, vp, i64, i32, vp, vp, vp, sz, vp]),
        "dflash_timing_enable": (C.c_int, [C.c_int]),
        "dflash_timing_read": (C.c_int, [i32, C.POINTER(i64), C.POINTER(C.c_double)]),
        "dflash_timing_reset": (C.c_int, []),
        "dflash_gemm_plan": (C.c_int, [C.c_int64, C.c_int64, C.c_int64, C.c_int32, C.POINTER(C.c_int32)]),
        "dflash_accept": (C.c_int, [vp, vp, i64, i32, vp, vp, vp, vp]),
        "dflash_attn_plan": (C.c_int, [C.POINTER(C.c_int64), i32, i32, i64, i32, C.POINTER(C.c_int64)]),
        "dflash_attn_force_chunk": (C.c_int, [i64]),
        "dflash_attn_sync_timeouts": (C.c_int, [vp]),
        "dflash_attn_force_merge_spread": (C.c_int, [i32]),
        "dflash_attn_set_spin_limit": (C.c_int, [i32]),
        "dflash_stream_read": (C.c_int, [vp, i64, vp, vp]),
        "dflash_mfma_peak": (C.c_int, [i32, i64, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


LIB = _load()


def strerror(code: int) -> str:
    return LIB.dflash_strerror(code).decode()


def _check(code: int, where: str) -> None:
    if code != DFLASH_OK:
        raise DFlashError(code, where)


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return DFLASH_F32
    if dt == torch.bfloat16:
        return DFLASH_BF16
    if dt == torch.float8_e4m3fn:
        return DFLASH_FP8_E4M3
    raise DFlashError(ERR_DTYPE, f"dtype {dt}")


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not (t.is_cuda and t.is_contiguous()):
        raise DFlashError(ERR_ARG, "tensors must be contiguous device tensors")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _i32(values):
    arr = (C.c_int32 * len(values))(*[int(v) for v in values])
    return arr


# --------------------------------------------------------------------- cache

class Cache:
    """dflash_cache handle plus the caller-owned device pools it describes."""

    def __init__(self, n_seqs, n_kv, d_h, dtype, capacity, page_size=0, max_pages_per_seq=0,
                 device="cuda", pools=None, ring=False, k_scale=1.0, v_scale=1.0):
        """dtype torch.float8_e4m3fn keeps K/V as E4M3 bytes (pools of
        torch.uint8 holding the codes) read as code value * k_scale / v_scale."""
        self.n_seqs, self.n_kv, self.d_h = n_seqs, n_kv, d_h
        self.page_size, self.capacity, self.max_pages = page_size, capacity, max_pages_per_seq
        self.ring = bool(ring)
        self.dtype = dtype
        self.fp8 = dtype == torch.float8_e4m3fn
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        pool_dt = torch.uint8 if self.fp8 else dtype
        if pools is not None:
            self.k_pool, self.v_pool, self.table = pools
        elif page_size == 0:
            self.k_pool = torch.zeros((n_seqs, n_kv, capacity, d_h), dtype=pool_dt, device=device)
            # V transposed in tiles of 64 slots: [.., tile, head dim, slot % 64]
            self.v_pool = torch.zeros((n_seqs, n_kv, -(-capacity // 64), d_h, 64), dtype=pool_dt, device=device)
            self.table = None
        else:
            self.k_pool = torch.zeros((capacity, n_kv, page_size, d_h), dtype=pool_dt, device=device)
            self.v_pool = torch.zeros((capacity, n_kv, -(-page_size // 64), d_h, 64), dtype=pool_dt, device=device)
            self.table = torch.full((n_seqs, max_pages_per_seq), -1, dtype=torch.int32, device=device)
        desc = CacheDesc(n_seqs, n_kv, d_h, dtype_code(dtype), page_size, max_pages_per_seq, 1 if ring else 0,
                         capacity,
                         self.k_pool.data_ptr(), self.v_pool.data_ptr(),
                         self.table.data_ptr() if self.table is not None else None,
                         self.k_scale, self.v_scale)
        h = C.c_void_p()
        _check(LIB.dflash_cache_init(C.byref(h), C.byref(desc)), "dflash_cache_init")
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        # at interpreter exit the module's globals may already be gone; the
        # handle's host memory goes with the process then
        if h is not None and h.value and LIB is not None:
            LIB.dflash_cache_destroy(h)
            self.handle = None

    def lengths(self):
        out = (C.c_int32 * self.n_seqs)()
        _check(LIB.dflash_cache_lengths(self.handle, out), "dflash_cache_lengths")
        return list(out)

    def block_table(self):
        mp = self.max_pages if self.page_size > 0 else 1
        out = (C.c_int32 * (self.n_seqs * mp))()
        _check(LIB.dflash_cache_block_table(self.handle, out), "dflash_cache_block_table")
        return [list(out[s * mp:(s + 1) * mp]) for s in range(self.n_seqs)]

    def free_pages(self) -> int:
        return int(LIB.dflash_cache_free_pages(self.handle))


def dflash_cache_append(cache: Cache, cu_rows, k_rows, v_rows, stream=None) -> None:
    """k_rows, v_rows: [rows, n_kv, d_h] device tensors of the cache's element
    size (E4M3 bytes as uint8 or float8_e4m3fn for fp8 caches).  The sizes are
    checked here: the C call can only trust its pointers."""
    rows = int(cu_rows[-1])
    if rows:
        esize = 1 if cache.fp8 else torch.empty((), dtype=cache.dtype).element_size()
        need = rows * cache.n_kv * cache.d_h
        for t in (k_rows, v_rows):
            if t is None or t.element_size() != esize or t.numel() < need:
                raise DFlashError(ERR_ARG, "dflash_cache_append: k_rows / v_rows must hold "
                                           f"[{rows}, {cache.n_kv}, {cache.d_h}] elements of {esize} byte(s)")
    _check(LIB.dflash_cache_append(cache.handle, _i32(cu_rows), _ptr(k_rows), _ptr(v_rows), _stream(stream)),
           "dflash_cache_append")


def dflash_cache_crop(cache: Cache, new_len, stream=None) -> None:
    _check(LIB.dflash_cache_crop(cache.handle, _i32(new_len), _stream(stream)), "dflash_cache_crop")


# --------------------------------------------------------------------- context projection

def dflash_ctx_project_ws_bytes(T, kd, d, dtype: torch.dtype) -> int:
    return int(LIB.dflash_ctx_project_ws_bytes(T, kd, d, dtype_code(dtype)))


def dflash_ctx_project(x_raw, w_fc, gamma_h, eps, c_out, ws, stream=None) -> None:
    T, kd = x_raw.shape
    d = w_fc.shape[0]
    _check(LIB.dflash_ctx_project(_ptr(x_raw), T, kd, _ptr(w_fc), _ptr(gamma_h), d, float(eps),
                                  dtype_code(x_raw.dtype), _ptr(c_out), _ptr(ws), ws.numel() if ws is not None else 0,
                                  _stream(stream)),
           "dflash_ctx_project")


# --------------------------------------------------------------------- layer

class Layer:
    """Device weights of one KV-injection attention layer and its descriptor."""

    def __init__(self, w_qkv, w_o, gamma_q, gamma_k, n_h, n_kv, d_h, eps=1e-6, rope_theta=1e6, window=0,
                 residual=False):
        self.w_qkv, self.w_o, self.gamma_q, self.gamma_k = w_qkv, w_o, gamma_q, gamma_k
        self.d = w_qkv.shape[1]
        self.desc = LayerDesc(self.d, n_h, n_kv, d_h, float(eps), float(rope_theta), int(window),
                              dtype_code(w_qkv.dtype), 1 if residual else 0, w_qkv.data_ptr(), w_o.data_ptr(),
                              gamma_q.data_ptr(), gamma_k.data_ptr())


def dflash_kv_inject_attn_ws_bytes(layer: Layer, cache: Cache, T: int, B: int) -> int:
    return int(LIB.dflash_kv_inject_attn_ws_bytes(C.byref(layer.desc), cache.handle, T, B))


def dflash_kv_inject_attn(layer: Layer, cache: Cache, C_rows, cu_ctx, H, B, out, ws, stream=None) -> None:
    _check(LIB.dflash_kv_inject_attn(C.byref(layer.desc), cache.handle, _ptr(C_rows) if C_rows is not None and C_rows.numel() else None,
                                     _i32(cu_ctx), _ptr(H), int(B), _ptr(out), _ptr(ws),
                                     ws.numel() if ws is not None else 0, _stream(stream)),
           "dflash_kv_inject_attn")


def dflash_kv_inject_attn_noalloc(layer: Layer, cache: Cache, C_rows, cu_ctx, H, B, out, stream=None) -> None:
    """The layer call with the library's own per-GPU scratch buffer instead of
    a caller workspace (allocates nothing)."""
    _check(LIB.dflash_kv_inject_attn_noalloc(C.byref(layer.desc), cache.handle,
                                             _ptr(C_rows) if C_rows is not None and C_rows.numel() else None,
                                             _i32(cu_ctx), _ptr(H), int(B), _ptr(out), _stream(stream)),
           "dflash_kv_inject_attn_noalloc")


# --------------------------------------------------------------------- device-driven rounds

def dflash_cache_device_begin(cache: Cache, d_len, stream=None) -> None:
    """Device mode: the cache's lengths live in d_len (int32 [n_seqs] device tensor)."""
    _check(LIB.dflash_cache_device_begin(cache.handle, _ptr(d_len), _stream(stream)), "dflash_cache_device_begin")


def dflash_kv_inject_attn_dev_ws_bytes(layer: Layer, cache: Cache, n_max: int, B: int) -> int:
    return int(LIB.dflash_kv_inject_attn_dev_ws_bytes(C.byref(layer.desc), cache.handle, int(n_max), int(B)))


def dflash_kv_inject_attn_dev(layer: Layer, cache: Cache, C_rows, n_max, d_rows, H, B, out, ws, stream=None) -> None:
    """A device-driven round: C_rows [n_seqs * n_max, d], d_rows int32 [n_seqs] device tensor."""
    _check(LIB.dflash_kv_inject_attn_dev(C.byref(layer.desc), cache.handle, _ptr(C_rows), int(n_max), _ptr(d_rows),
                                         _ptr(H), int(B), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)),
           "dflash_kv_inject_attn_dev")


def dflash_cache_crop_tail_dev(cache: Cache, drop: int, stream=None) -> None:
    _check(LIB.dflash_cache_crop_tail_dev(cache.handle, int(drop), _stream(stream)), "dflash_cache_crop_tail_dev")


def dflash_cache_device_reset(cache: Cache, host_len, stream=None) -> None:
    """Device-side lengths set back to host_len (each at most the host bound)."""
    _check(LIB.dflash_cache_device_reset(cache.handle, _i32(host_len), _stream(stream)), "dflash_cache_device_reset")


def dflash_cache_device_end(cache: Cache, stream=None) -> None:
    """Leave device mode (synchronises the stream and reads the lengths back)."""
    _check(LIB.dflash_cache_device_end(cache.handle, _stream(stream)), "dflash_cache_device_end")


# --------------------------------------------------------------------- draft head

def dflash_draft_head_ws_bytes(R, B, d, vocab, dtype: torch.dtype) -> int:
    return int(LIB.dflash_draft_head_ws_bytes(R, B, d, vocab, dtype_code(dtype)))


def dflash_draft_head(h, B, gamma_f, eps, w_lm, token_ids, ws, max_logit=None, stream=None) -> None:
    """h [R*B, d]; token_ids [R*(B-1)] int32 (and max_logit float32) device tensors."""
    RB, d = h.shape
    vocab = w_lm.shape[0]
    _check(LIB.dflash_draft_head(_ptr(h), RB // B, int(B), d, _ptr(gamma_f), float(eps), _ptr(w_lm), vocab,
                                 dtype_code(h.dtype), _ptr(token_ids), _ptr(max_logit), _ptr(ws),
                                 ws.numel() if ws is not None else 0, _stream(stream)),
           "dflash_draft_head")


def dflash_accept(draft_ids, posterior, acc, next_rows=None, next_anchor=None, stream=None) -> None:
    """posterior [R, B] int32; draft_ids [R*(B-1)] (or [R, B-1]) int32; acc,
    next_rows, next_anchor [R] int32 device tensors (the last two optional)."""
    R, B = posterior.shape
    _check(LIB.dflash_accept(_ptr(draft_ids), _ptr(posterior), int(R), int(B), _ptr(acc), _ptr(next_rows),
                             _ptr(next_anchor), _stream(stream)), "dflash_accept")


# --------------------------------------------------------------------- stage timing

STAGES = ("ctx_gemm", "ctx_reduce", "ctx_norm", "qkv_gemm", "qkv_epilogue", "attn", "attn_combine",
          "o_gemm", "o_reduce", "cache_append", "page_table", "head_norm", "head_gemm", "head_argmax",
          "accept", "stream_read", "mfma_peak")


def timing_enable(on: bool = True) -> None:
    _check(LIB.dflash_timing_enable(1 if on else 0), "dflash_timing_enable")


def timing_reset() -> None:
    _check(LIB.dflash_timing_reset(), "dflash_timing_reset")


GEMM_KERNELS = ("lds", "wide", "stream", "fullk", "resident", "slab", "tile")


def dflash_gemm_plan(M: int, N: int, K: int, dtype) -> dict:
    """The kernel and decomposition the library picks for a product of M rows
    with an [N][K] weight (host-side planning only)."""
    out = (C.c_int32 * 6)()
    _check(LIB.dflash_gemm_plan(int(M), int(N), int(K), dtype_code(dtype), out), "dflash_gemm_plan")
    return {"kernel": GEMM_KERNELS[out[0]], "splits": out[1], "k_chunk": out[2], "n_tiles": out[3],
            "tile_bn": out[4], "rows_per_problem": out[5]}


def dflash_attn_plan(keys, n_kv: int, chunk_cap: int = 1 << 30, cache_dtype: int = DFLASH_BF16) -> dict:
    """The attention split a layer call would use for these per-sequence key
    counts (host-side planning only)."""
    k = (C.c_int64 * len(keys))(*[int(x) for x in keys])
    out = (C.c_int64 * 3)()
    _check(LIB.dflash_attn_plan(k, len(keys), int(n_kv), int(chunk_cap), int(cache_dtype), out),
           "dflash_attn_plan")
    return {"chunk": int(out[0]), "items": int(out[1]), "nst": int(out[2])}


def dflash_stream_read(t, stream=None) -> None:
    """A plain streaming read of the bytes of device tensor t (measurement)."""
    _check(LIB.dflash_stream_read(_ptr(t), t.numel() * t.element_size(), None, _stream(stream)), "dflash_stream_read")


def dflash_mfma_peak(iters: int, workgroups: int, stream=None) -> None:
    """Back-to-back bf16 MFMAs on register operands (measurement): 8 * iters
    16x16x32 products per wave, four waves per workgroup."""
    _check(LIB.dflash_mfma_peak(int(iters), int(workgroups), None, _stream(stream)), "dflash_mfma_peak")


def dflash_attn_force_chunk(chunk: int) -> None:
    """Force the attention split of later layer calls to `chunk` keys per
    item (0: the planner's split); a diagnostic for split-invariance tests."""
    _check(LIB.dflash_attn_force_chunk(int(chunk)), "dflash_attn_force_chunk")


def dflash_attn_force_merge_spread(on: bool) -> None:
    """Deal each K/V head's attention items to consecutive workgroups where the
    split merges in the attention launch (a diagnostic: the merge then takes
    its write-back path across XCDs)."""
    _check(LIB.dflash_attn_force_merge_spread(1 if on else 0), "dflash_attn_force_merge_spread")


ATTN_SPIN_LIMIT = 1 << 18


def dflash_attn_set_spin_limit(polls: int) -> None:
    """Polls before an in-launch merge wait gives up (0: at once; the default
    ATTN_SPIN_LIMIT restores ordinary calls); a diagnostic for tests of the
    time-out path."""
    _check(LIB.dflash_attn_set_spin_limit(int(polls)), "dflash_attn_set_spin_limit")


def dflash_attn_sync_timeouts() -> int:
    """Attention workgroups whose in-launch merge wait timed out on the
    current device since the library was loaded (0 in every correct run)."""
    n = C.c_uint32(0)
    _check(LIB.dflash_attn_sync_timeouts(C.byref(n)), "dflash_attn_sync_timeouts")
    return int(n.value)


def timing_read() -> dict:
    """{stage name: (launches, total ms)} since the last reset."""
    out = {}
    for i, name in enumerate(STAGES):
        n, ms = C.c_int64(), C.c_double()
        _check(LIB.dflash_timing_read(i, C.byref(n), C.byref(ms)), "dflash_timing_read")
        out[name] = (int(n.value), float(ms.value))
    return out
