"""C-ABI contract checks that need no GPU: the library loads and exports every
symbol of include/dflash.h, the ctypes structs match the C layout, and every
validation path returns its documented status before anything is enqueued
(fake, never-dereferenced device pointers)."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")

L = pytest.importorskip("block_diffusion_draft_fc_amd._lib")

FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation or touches host state only


def test_exports_every_declared_symbol():
    names = set(re.findall(r"\b(dflash_\w+)\s*\(", open(HEADER).read()))
    assert {"dflash_ctx_project", "dflash_kv_inject_attn", "dflash_cache_append", "dflash_cache_crop"} <= names
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dflash_\w+)", out))
    assert names <= exported, names - exported


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "dflash.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(dflash_layer_desc), offsetof(dflash_layer_desc, eps),
         offsetof(dflash_layer_desc, rope_theta), offsetof(dflash_layer_desc, window),
         offsetof(dflash_layer_desc, residual), offsetof(dflash_layer_desc, gamma_k));
  printf("%zu %zu %zu %zu %zu %zu %zu\\n", sizeof(dflash_cache_desc), offsetof(dflash_cache_desc, capacity),
         offsetof(dflash_cache_desc, k_pool), offsetof(dflash_cache_desc, block_table),
         offsetof(dflash_cache_desc, ring), offsetof(dflash_cache_desc, k_scale),
         offsetof(dflash_cache_desc, v_scale));
  return 0;
}""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    ld, cd = L.LayerDesc, L.CacheDesc
    assert [int(x) for x in lines[0].split()] == [C.sizeof(ld), ld.eps.offset, ld.rope_theta.offset,
                                                  ld.window.offset, ld.residual.offset, ld.gamma_k.offset]
    assert [int(x) for x in lines[1].split()] == [C.sizeof(cd), cd.capacity.offset, cd.k_pool.offset,
                                                  cd.block_table.offset, cd.ring.offset, cd.k_scale.offset,
                                                  cd.v_scale.offset]


def _cache(n_seqs=2, page_size=0, capacity=128, max_pages=0, dtype=L.DFLASH_BF16, ring=0, k_scale=1.0,
           v_scale=1.0):
    desc = L.CacheDesc(n_seqs, 2, 64, dtype, page_size, max_pages, ring, capacity, FAKE, FAKE,
                       FAKE if page_size else None, k_scale, v_scale)
    h = C.c_void_p()
    rc = L.LIB.dflash_cache_init(C.byref(h), C.byref(desc))
    return rc, h


def test_strerror_table():
    for code in range(0, -8, -1):
        assert L.strerror(code) and L.strerror(code) != "unknown status"
    assert L.strerror(-99) == "unknown status"


@pytest.mark.parametrize("kw,code", [
    (dict(capacity=100), L.ERR_SHAPE),                 # contiguous capacity not a multiple of 64
    (dict(page_size=100, capacity=4, max_pages=4), L.ERR_SHAPE),
    (dict(page_size=64, capacity=4, max_pages=0), L.ERR_SHAPE),
    (dict(n_seqs=0), L.ERR_SHAPE),
    (dict(n_seqs=65), L.ERR_SHAPE),
    (dict(dtype=7), L.ERR_DTYPE),
    (dict(page_size=64, capacity=4, max_pages=4, ring=1), L.ERR_SHAPE),   # rings are contiguous only
    (dict(ring=2), L.ERR_SHAPE),
    (dict(dtype=L.DFLASH_FP8_E4M3, k_scale=0.0), L.ERR_ARG),     # fp8 scales finite and > 0
    (dict(dtype=L.DFLASH_FP8_E4M3, v_scale=-1.0), L.ERR_ARG),
    (dict(dtype=L.DFLASH_FP8_E4M3, v_scale=float("nan")), L.ERR_ARG),
    (dict(dtype=L.DFLASH_FP8_E4M3, k_scale=float("inf")), L.ERR_ARG),
    (dict(dtype=L.DFLASH_BF16, k_scale=0.0), L.DFLASH_OK),       # other dtypes ignore the scales
    (dict(dtype=L.DFLASH_FP8_E4M3, k_scale=0.5, v_scale=3.0), L.DFLASH_OK),
])
def test_cache_init_rejects(kw, code):
    rc, h = _cache(**kw)
    assert rc == code
    if rc == L.DFLASH_OK:
        L.LIB.dflash_cache_destroy(h)


def test_cache_host_metadata_and_errors():
    rc, h = _cache(n_seqs=2, page_size=64, capacity=3, max_pages=2)
    assert rc == L.DFLASH_OK
    try:
        lens = (C.c_int32 * 2)()
        assert L.LIB.dflash_cache_lengths(h, lens) == 0 and list(lens) == [0, 0]
        assert L.LIB.dflash_cache_free_pages(h) == 3
        # crop beyond the current length
        assert L.LIB.dflash_cache_crop(h, L._i32([1, 0]), None) == L.ERR_RANGE
        assert L.LIB.dflash_cache_crop(h, L._i32([0, 0]), None) == L.DFLASH_OK
        # malformed offsets
        assert L.LIB.dflash_cache_append(h, L._i32([1, 2, 3]), FAKE, FAKE, None) == L.ERR_ARG
        assert L.LIB.dflash_cache_append(h, L._i32([0, 5, 3]), FAKE, FAKE, None) == L.ERR_ARG
        # 129 rows need 3 pages > max_pages_per_seq = 2
        assert L.LIB.dflash_cache_append(h, L._i32([0, 129, 129]), FAKE, FAKE, None) == L.ERR_CAPACITY
        # 2 + 2 pages > pool of 3
        assert L.LIB.dflash_cache_append(h, L._i32([0, 128, 256]), FAKE, FAKE, None) == L.ERR_CAPACITY
        # misaligned rows
        assert L.LIB.dflash_cache_append(h, L._i32([0, 1, 1]), FAKE + 2, FAKE, None) == L.ERR_ARG
        # a zero-row append is a no-op that succeeds without touching the device
        assert L.LIB.dflash_cache_append(h, L._i32([0, 0, 0]), None, None, None) == L.DFLASH_OK
        assert L.LIB.dflash_cache_lengths(h, lens) == 0 and list(lens) == [0, 0]
        assert L.LIB.dflash_cache_free_pages(h) == 3
        tab = (C.c_int32 * 4)()
        assert L.LIB.dflash_cache_block_table(h, tab) == 0 and list(tab) == [-1] * 4
    finally:
        L.LIB.dflash_cache_destroy(h)


def test_contiguous_capacity_error():
    rc, h = _cache(n_seqs=1, capacity=64)
    assert rc == 0
    try:
        assert L.LIB.dflash_cache_append(h, L._i32([0, 65]), FAKE, FAKE, None) == L.ERR_CAPACITY
        tab = (C.c_int32 * 1)()
        assert L.LIB.dflash_cache_block_table(h, tab) == 0 and list(tab) == [0]
    finally:
        L.LIB.dflash_cache_destroy(h)


def test_ctx_project_validation():
    f = L.LIB.dflash_ctx_project
    ws = L.LIB.dflash_ctx_project_ws_bytes(16, 20480, 4096, L.DFLASH_BF16)
    assert ws >= 16 * 4096 * 4
    assert L.LIB.dflash_ctx_project_ws_bytes(0, 20480, 4096, L.DFLASH_BF16) == 0
    # T = 0 is a no-op
    assert f(None, 0, 1536, None, None, 512, 1e-6, L.DFLASH_F32, None, None, 0, None) == 0
    assert f(FAKE, 3, 1536, FAKE, FAKE, 512, 1e-6, 5, FAKE, FAKE, 1 << 30, None) == L.ERR_DTYPE
    assert f(FAKE, 3, 1535, FAKE, FAKE, 512, 1e-6, 0, FAKE, FAKE, 1 << 30, None) == L.ERR_SHAPE
    assert f(None, 3, 1536, FAKE, FAKE, 512, 1e-6, 0, FAKE, FAKE, 1 << 30, None) == L.ERR_ARG
    assert f(FAKE + 4, 3, 1536, FAKE, FAKE, 512, 1e-6, 0, FAKE, FAKE, 1 << 30, None) == L.ERR_ARG
    assert f(FAKE, 3, 1536, FAKE, FAKE, 512, 1e-6, 0, FAKE, FAKE, 16, None) == L.ERR_WORKSPACE


def _layer(**kw):
    base = dict(d=512, n_h=8, n_kv=2, d_h=64, eps=1e-6, rope_theta=1e6, window=0, dtype=L.DFLASH_BF16)
    base.update(kw)
    return L.LayerDesc(base["d"], base["n_h"], base["n_kv"], base["d_h"], base["eps"], base["rope_theta"],
                       base["window"], base["dtype"], base.get("residual", 0), FAKE, FAKE, FAKE, FAKE)


def test_kv_inject_validation():
    rc, h = _cache(n_seqs=2, capacity=128)
    assert rc == 0
    try:
        f = L.LIB.dflash_kv_inject_attn
        good = _layer()
        wsb = L.LIB.dflash_kv_inject_attn_ws_bytes(C.byref(good), h, 8, 4)
        assert wsb > 0
        cu = L._i32([0, 4, 8])
        args = lambda lay, B=4, cu=cu, ws=wsb: (C.byref(lay), h, FAKE, cu, FAKE, B, FAKE, FAKE, ws, None)  # noqa: E731
        assert f(*args(_layer(dtype=L.DFLASH_F32))) == L.ERR_DTYPE          # cache is bf16
        assert f(*args(_layer(n_kv=4, n_h=8))) == L.ERR_SHAPE                # cache has 2 K/V heads
        assert f(*args(_layer(n_h=7))) == L.ERR_SHAPE                        # n_h % n_kv
        assert f(*args(_layer(d_h=96))) == L.ERR_SHAPE
        assert f(*args(good, B=17)) == L.ERR_SHAPE                           # group 4 * 17 > 64 rows
        assert f(*args(good, cu=L._i32([0, 9, 8]))) == L.ERR_ARG
        assert f(*args(good, ws=wsb - 1)) == L.ERR_WORKSPACE
        # 64 + 64 + 4 rows exceed the 128-row capacity
        ws_big = L.LIB.dflash_kv_inject_attn_ws_bytes(C.byref(good), h, 126, 4)
        assert f(*args(good, cu=L._i32([0, 125, 126]), ws=ws_big)) == L.ERR_CAPACITY
        lens = (C.c_int32 * 2)()
        L.LIB.dflash_cache_lengths(h, lens)
        assert list(lens) == [0, 0]
    finally:
        L.LIB.dflash_cache_destroy(h)


def test_fp8_cache_needs_a_bf16_layer():
    rc, h = _cache(n_seqs=2, capacity=128, dtype=L.DFLASH_FP8_E4M3, k_scale=0.25, v_scale=2.0)
    assert rc == 0
    try:
        f = L.LIB.dflash_kv_inject_attn
        good = _layer()
        wsb = L.LIB.dflash_kv_inject_attn_ws_bytes(C.byref(good), h, 8, 4)
        assert wsb > 0
        cu = L._i32([0, 4, 8])
        args = lambda lay, ws=wsb: (C.byref(lay), h, FAKE, cu, FAKE, 4, FAKE, FAKE, ws, None)  # noqa: E731
        assert f(*args(_layer(dtype=L.DFLASH_F32))) == L.ERR_DTYPE
        assert f(*args(_layer(dtype=L.DFLASH_FP8_E4M3))) == L.ERR_DTYPE     # not a layer dtype
        assert f(*args(good, ws=wsb - 1)) == L.ERR_WORKSPACE                 # past the dtype checks
    finally:
        L.LIB.dflash_cache_destroy(h)


def test_ring_validation():
    """Ring caches: lengths beyond the capacity are allowed, one call brings at
    most `capacity` rows per sequence, and a layer call needs a sliding window
    with window + B - 1 <= capacity and n + B <= capacity."""
    rc, h = _cache(n_seqs=2, capacity=128, ring=1)
    assert rc == 0
    try:
        # 129 rows in one call would land twice in one slot
        assert L.LIB.dflash_cache_append(h, L._i32([0, 129, 129]), FAKE, FAKE, None) == L.ERR_CAPACITY
        f = L.LIB.dflash_kv_inject_attn

        def call(lay, cu, B=4):
            ws = L.LIB.dflash_kv_inject_attn_ws_bytes(C.byref(lay), h, cu[-1], B)
            return f(C.byref(lay), h, FAKE, L._i32(cu), FAKE, B, FAKE, FAKE, ws, None)

        assert call(_layer(window=0), [0, 4, 8]) == L.ERR_SHAPE            # full attention on a ring
        assert call(_layer(window=126), [0, 4, 8]) == L.ERR_CAPACITY       # 126 + 4 - 1 > 128
        assert call(_layer(window=100), [0, 125, 126]) == L.ERR_CAPACITY   # 125 + 4 new rows > 128
        lens = (C.c_int32 * 2)()
        L.LIB.dflash_cache_lengths(h, lens)
        assert list(lens) == [0, 0]
    finally:
        L.LIB.dflash_cache_destroy(h)


def test_workspace_figures_cover_every_smaller_call():
    """A workspace sized for T rows serves every call with fewer rows, although
    the projection plans (one fused q/k/v product up to 64 rows, split counts)
    change with the rows."""
    rc, h = _cache(n_seqs=3, capacity=512)
    assert rc == 0
    try:
        lay = _layer(d=256, n_h=8, n_kv=2, d_h=128)
        f = lambda T: L.LIB.dflash_kv_inject_attn_ws_bytes(C.byref(lay), h, T, 16)  # noqa: E731
        figs = [f(T) for T in range(0, 80)]
        assert all(b >= a for a, b in zip(figs, figs[1:])), figs
        g = lambda T: L.LIB.dflash_ctx_project_ws_bytes(T, 20480, 4096, L.DFLASH_BF16)  # noqa: E731
        figs = [g(T) for T in range(1, 80)]
        assert all(b >= a for a, b in zip(figs, figs[1:])), figs
    finally:
        L.LIB.dflash_cache_destroy(h)


def test_draft_head_validation():
    f = L.LIB.dflash_draft_head
    ws = L.LIB.dflash_draft_head_ws_bytes(1, 16, 4096, 151936, L.DFLASH_BF16)
    assert ws >= 15 * 151936 * 4
    assert L.LIB.dflash_draft_head_ws_bytes(1, 1, 4096, 151936, L.DFLASH_BF16) == 0
    args = lambda R=1, B=16, d=512, vocab=1000, dt=L.DFLASH_BF16, ids=FAKE, w=1 << 30: (  # noqa: E731
        FAKE, R, B, d, FAKE, 1e-6, FAKE, vocab, dt, ids, None, FAKE, w, None)
    assert f(*args(dt=9)) == L.ERR_DTYPE
    assert f(*args(vocab=1002)) == L.ERR_SHAPE          # vocab % 4
    assert f(*args(d=500)) == L.ERR_SHAPE               # d % 8
    assert f(*args(R=0)) == L.ERR_SHAPE
    assert f(*args(ids=None)) == L.ERR_ARG
    assert f(*args(ids=FAKE + 2)) == L.ERR_ARG
    assert f(*args(w=16)) == L.ERR_WORKSPACE
    assert f(*args(B=1, ids=None)) == L.DFLASH_OK       # nothing to predict


# ------------------------------------------------------------------ GEMM plans (host-side planning)

def _plan(M, N, K, dt):
    out = (C.c_int32 * 6)()
    rc = L.LIB.dflash_gemm_plan(M, N, K, dt, out)
    return rc, {"kernel": L.GEMM_KERNELS[out[0]] if rc == 0 else None, "splits": out[1], "k_chunk": out[2],
                "n_tiles": out[3], "tile_bn": out[4], "rows_per_problem": out[5]}


# the projections of the named workloads and the kernel each takes: decode
# rounds (<= 16 and <= 32 rows), the 4-request stack (64 block rows, up to 128
# [C; H] rows), the 16-request ragged batch (256 block rows, ~400 [C; H] rows),
# the fresh 1024-row context and the draft head over the Qwen3 vocabulary
ROUTES = [
    ((16, 4096, 20480), "fullk"), ((16, 4096, 4096), "fullk"), ((32, 6144, 4096), "stream"),
    ((24, 6144, 4096), "stream"), ((64, 4096, 4096), "stream"), ((128, 2048, 4096), "slab"),
    ((48, 4096, 20480), "slab"), ((100, 4096, 20480), "tile"), ((256, 4096, 4096), "tile"),
    ((392, 2048, 4096), "tile"), ((1024, 2560, 12800), "tile"), ((15, 151936, 4096), "resident"),
    ((20, 4096, 20480), "wide"),
]


@pytest.mark.parametrize("shape,kernel", ROUTES, ids=[f"{m}x{n}x{k}" for (m, n, k), _ in ROUTES])
def test_gemm_plan_routes(shape, kernel):
    rc, p = _plan(*shape, L.DFLASH_BF16)
    assert rc == 0 and p["kernel"] == kernel, p


def test_gemm_plan_invariants():
    """Over a grid of shapes: the splits cover K exactly once in whole chunks,
    every kernel's own limits hold (rows, K alignment, LDS budget, tile width),
    and the fp32 path stays on the kernel that handles it."""
    for dt in (L.DFLASH_BF16, L.DFLASH_F32):
        for M in (1, 3, 16, 17, 31, 32, 33, 48, 63, 64, 65, 100, 128, 129, 200, 256, 300, 1040):
            for N in (64, 520, 2048, 4096, 6144, 70000):
                for K in (256, 512, 1536, 2080, 4096, 12800, 20480):
                    rc, p = _plan(M, N, K, dt)
                    assert rc == 0, (M, N, K, dt)
                    kind, sp, kc = p["kernel"], p["splits"], p["k_chunk"]
                    where = (M, N, K, dt, p)
                    assert sp >= 1 and kc >= 1 and (sp - 1) * kc < K <= sp * kc, where
                    if dt == L.DFLASH_F32:
                        assert kind == "lds" and p["rows_per_problem"] == 32, where
                        continue
                    rows = min(M, p["rows_per_problem"]) if kind != "tile" else M
                    if kind in ("fullk", "resident"):
                        assert rows <= 16 and sp == 1 and kc == K, where
                    if kind == "wide":
                        assert rows <= 32, where
                    if kind == "stream":
                        assert rows <= 64 and K < 8192 and K % 64 == 0 and kc == 512, where
                        waves = 12 if -(-rows // 16) == 2 else 8
                        assert p["n_tiles"] == -(-N // (16 * waves)), where
                    if kind == "slab":
                        mt = -(-rows // 16)
                        assert 3 <= mt <= 8 and K % 512 == 0 and kc % 512 == 0, where
                        assert mt >= 5 or K >= 8192, where
                        assert mt * 16 * (kc + 8) * 2 <= 160 * 1024, where
                        assert p["n_tiles"] == -(-N // 64), where
                    if kind == "tile":
                        assert p["tile_bn"] in (64, 128, 256) and kc % 64 == 0, where
                        assert p["n_tiles"] == -(-N // p["tile_bn"]), where
                        assert M > p["rows_per_problem"] or p["rows_per_problem"] == 0, where
                    if kind == "lds":
                        assert kc % 256 == 0 and -(-rows // 16) * 16 * (kc + 8) * 2 <= 64 * 1024, where


def test_gemm_plan_validation():
    out = (C.c_int32 * 6)()
    assert L.LIB.dflash_gemm_plan(16, 64, 64, L.DFLASH_BF16, None) == L.ERR_ARG
    assert L.LIB.dflash_gemm_plan(0, 64, 64, L.DFLASH_BF16, out) == L.ERR_SHAPE
    assert L.LIB.dflash_gemm_plan(16, 0, 64, L.DFLASH_BF16, out) == L.ERR_SHAPE
    assert L.LIB.dflash_gemm_plan(16, 64, -1, L.DFLASH_BF16, out) == L.ERR_SHAPE
    assert L.LIB.dflash_gemm_plan(16, 64, 64, 7, out) == L.ERR_DTYPE


def test_accept_validation():
    f = L.LIB.dflash_accept
    assert f(FAKE, FAKE, 4, 0, FAKE, None, None, None) == L.ERR_SHAPE        # B < 1
    assert f(FAKE, FAKE, -1, 16, FAKE, None, None, None) == L.ERR_SHAPE      # R < 0
    assert f(FAKE, FAKE, 1 << 31, 16, FAKE, None, None, None) == L.ERR_SHAPE
    assert f(FAKE, FAKE, 4, 16, None, None, None, None) == L.ERR_ARG         # acc missing
    assert f(FAKE, None, 4, 16, FAKE, None, None, None) == L.ERR_ARG         # posterior missing
    assert f(None, FAKE, 4, 16, FAKE, None, None, None) == L.ERR_ARG         # draft missing, B > 1
    assert f(FAKE + 2, FAKE, 4, 16, FAKE, None, None, None) == L.ERR_ARG     # misaligned
    assert f(FAKE, FAKE, 4, 16, FAKE, FAKE, FAKE + 1, None) == L.ERR_ARG
    assert f(None, None, 0, 16, None, None, None, None) == L.DFLASH_OK       # no requests: no-op


# ------------------------------------------------------------------ attention split (host-side planning)

def _attn_plan(keys, n_kv, cap=1 << 30, dtype=L.DFLASH_BF16):
    k = (C.c_int64 * len(keys))(*keys)
    out = (C.c_int64 * 3)()
    rc = L.LIB.dflash_attn_plan(k, len(keys), n_kv, cap, dtype, out)
    return rc, int(out[0]), int(out[1]), int(out[2])


def _items(keys, n_kv, chunk):
    return sum(max(1, -(-k // chunk)) * n_kv for k in keys)


# key counts of the named workloads: one 8K decode round (8192 cached + 16
# block keys, plus the round's context rows), four 32K requests, a 4-request
# stack, a 16-request ragged batch, a 4096-key sliding window on a ring of
# 4096 + 64 rows, and a paged pool of 256-row pages
ATTN_CASES = [
    ([8216], 8, 1 << 30), ([8256], 8, 1 << 30), ([32792] * 4, 8, 1 << 30),
    ([1040, 2112, 4160, 8256], 8, 1 << 30),
    ([200 + 977 * i for i in range(16)], 8, 1 << 30), ([4160] * 4, 8, 62 * 4160),
    ([33024] * 4, 8, 62 * 256), ([64], 1, 1 << 30), ([1], 8, 1 << 30), ([1 << 20], 8, 62 * 256),
    ([100] * 64, 8, 1 << 30), ([300000] * 64, 8, 62 * 256), ([5000, 70, 130000], 2, 62 * 1024),
]


@pytest.mark.parametrize("dtype", [L.DFLASH_BF16, L.DFLASH_FP8_E4M3], ids=["bf16", "fp8"])
@pytest.mark.parametrize("keys,n_kv,cap", ATTN_CASES, ids=[f"{len(k)}x{max(k)}-kv{g}-cap{c}" for k, g, c in ATTN_CASES])
def test_attn_plan_invariants(keys, n_kv, cap, dtype):
    """The chunk is a whole number of 64-key blocks, at least 128 and within
    the cap; the item count is what the chunk gives; the ring depth follows the
    total key count; and the chunk is the smallest that brings the items into
    one round of launch slots (256 workgroups at depth 3, 512 at depth 2, 1024
    at depth 2 for fp8 caches), or the cap when no chunk within it does."""
    rc, chunk, items, nst = _attn_plan(keys, n_kv, cap, dtype)
    assert rc == 0
    total = sum(keys) * n_kv
    assert nst == (2 if total > 256 * 1024 else 3)
    capc = max(128, cap // 64 * 64)
    assert chunk % 64 == 0 and 128 <= chunk <= capc
    assert items == _items(keys, n_kv, chunk)
    limit = (1024 if dtype == L.DFLASH_FP8_E4M3 else 512) if nst == 2 else 256
    if _items(keys, n_kv, capc) <= limit:
        assert items <= limit
        assert chunk == 128 or _items(keys, n_kv, chunk - 64) > limit
    else:
        assert chunk == capc
    # the workspace sizes partials for at most 1024 items plus two per
    # (sequence, head), plus what a capped chunk adds
    assert items <= 1024 + 2 * len(keys) * n_kv + -(-total // (capc - 128 if capc > 128 else 64))


def test_attn_plan_headline_split():
    """The 8K decode round: 8 heads x 26 chunks of 320 keys, one round of 256
    slots at ring depth 3."""
    assert _attn_plan([8216], 8) == (0, 320, 208, 3)
    assert _attn_plan([8216], 8, dtype=L.DFLASH_FP8_E4M3) == (0, 320, 208, 3)
    # four 32K requests: 512 items for bf16, 992 for fp8 caches (chunks of 1088)
    assert _attn_plan([32792] * 4, 8)[2] == 512
    assert _attn_plan([32792] * 4, 8, dtype=L.DFLASH_FP8_E4M3)[1:3] == (1088, 992)


def test_device_mode_validation():
    """Device-driven rounds: a ring cannot enter device mode, a null or
    misaligned length array is refused, and the device-round calls need device
    mode; all checked before anything is enqueued."""
    rc, ring = _cache(ring=1)
    assert rc == 0
    assert L.LIB.dflash_cache_device_begin(ring, FAKE, None) == L.ERR_SHAPE
    rc, h = _cache()
    assert rc == 0
    assert L.LIB.dflash_cache_device_begin(h, None, None) == L.ERR_ARG
    assert L.LIB.dflash_cache_device_begin(h, C.c_void_p(FAKE + 2), None) == L.ERR_ARG
    assert L.LIB.dflash_cache_crop_tail_dev(h, 4, None) == L.ERR_ARG
    assert L.LIB.dflash_cache_device_end(h, None) == L.ERR_ARG
    lay = L.LayerDesc(512, 8, 2, 64, 1e-6, 1e6, 0, L.DFLASH_BF16, 0, FAKE, FAKE, FAKE, FAKE)
    f = L.LIB.dflash_kv_inject_attn_dev
    assert f(C.byref(lay), h, FAKE, 4, None, FAKE, 4, FAKE, FAKE, 1 << 30, None) == L.ERR_ARG
    assert f(C.byref(lay), h, FAKE, -1, FAKE, FAKE, 4, FAKE, FAKE, 1 << 30, None) == L.ERR_SHAPE
    # a cache in host mode takes no device-driven round
    assert f(C.byref(lay), h, FAKE, 4, FAKE, FAKE, 4, FAKE, FAKE, 1 << 30, None) == L.ERR_ARG
    assert L.LIB.dflash_kv_inject_attn_dev_ws_bytes(C.byref(lay), h, 4, 4) == \
        L.LIB.dflash_kv_inject_attn_ws_bytes(C.byref(lay), h, 8, 4)
    for c in (ring, h):
        L.LIB.dflash_cache_destroy(c)


def test_stream_read_validation():
    """The measurement read refuses negative sizes and misaligned sources
    before launching anything, and a zero-byte read is a no-op."""
    f = L.LIB.dflash_stream_read
    assert f(C.c_void_p(16), -1, None, None) == L.ERR_SHAPE
    assert f(C.c_void_p(8), 64, None, None) == L.ERR_ARG
    assert f(None, 64, None, None) == L.ERR_ARG
    assert f(C.c_void_p(16), 64, C.c_void_p(2), None) == L.ERR_ARG
    assert f(None, 0, None, None) == 0


def test_mfma_peak_validation():
    """The matrix-core probe refuses out-of-range sizes and misaligned sinks
    before launching anything."""
    f = L.LIB.dflash_mfma_peak
    for it, wg in ((0, 1), (1 << 25, 1), (1, 0), (1, (1 << 20) + 1)):
        assert f(it, wg, None, None) == L.ERR_SHAPE
    assert f(1, 1, C.c_void_p(2), None) == L.ERR_ARG


def test_attn_force_chunk():
    """The split override: multiples of 64 from 64 up, 0 restores the planner;
    the plan then reports the forced chunk (capped by the cache's limit)."""
    f = L.LIB.dflash_attn_force_chunk
    for bad in (-64, 32, 100, 1 << 31):
        assert f(bad) == L.ERR_SHAPE
    try:
        assert f(128) == 0
        assert _attn_plan([8216], 8) == (0, 128, 8 * 65, 3)
        assert _attn_plan([33024] * 4, 8, 62 * 64 * 1) == (0, 128, 4 * 8 * 258, 2)
        assert f(1 << 20) == 0
        assert _attn_plan([33024] * 4, 8, 62 * 256)[1:3] == (62 * 256, 4 * 8 * 3)   # capped at 62 pages
    finally:
        assert f(0) == 0
    assert _attn_plan([8216], 8) == (0, 320, 208, 3)


def test_attn_merge_diagnostics_validation():
    """The merge's item-order switch takes 0 or 1, its wait bound 0 .. 2^18
    polls; both only set process-wide values (no device call)."""
    spread = L.LIB.dflash_attn_force_merge_spread
    for bad in (-1, 2, 7):
        assert spread(bad) == L.ERR_ARG
    assert spread(0) == 0
    spin = L.LIB.dflash_attn_set_spin_limit
    for bad in (-1, (1 << 18) + 1, 1 << 30):
        assert spin(bad) == L.ERR_ARG
    try:
        assert spin(0) == 0 and spin(5) == 0
    finally:
        assert spin(L.ATTN_SPIN_LIMIT) == 0


def test_attn_plan_validation():
    k = (C.c_int64 * 2)(100, 200)
    out = (C.c_int64 * 3)()
    f = L.LIB.dflash_attn_plan
    bf = L.DFLASH_BF16
    assert f(None, 2, 8, 1 << 30, bf, out) == L.ERR_ARG
    assert f(k, 2, 8, 1 << 30, bf, None) == L.ERR_ARG
    assert f(k, 2, 8, 1 << 30, 9, out) == L.ERR_DTYPE
    assert f(k, 0, 8, 1 << 30, bf, out) == L.ERR_SHAPE
    assert f(k, 2, 0, 1 << 30, bf, out) == L.ERR_SHAPE
    assert f(k, 2, 8, 63, bf, out) == L.ERR_SHAPE
    z = (C.c_int64 * 2)(100, 0)
    assert f(z, 2, 8, 1 << 30, bf, out) == L.ERR_SHAPE
    assert L.dflash_attn_plan([100, 200], 8) == {"chunk": 128, "items": 24, "nst": 3}
