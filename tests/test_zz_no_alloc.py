"""GPU check of dflash_kv_inject_attn_noalloc (the layer call on the library's
own per-GPU scratch buffer, for callers that cannot allocate) against
dflash_kv_inject_attn on a caller workspace: two calls in a row on twin
caches, the second with fewer context rows, outputs and cache contents bit for
bit equal and within the bf16 bar of the fp64 oracle; a call too large for the
buffer is refused with nothing enqueued."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU visible", allow_module_level=True)

from block_diffusion_draft_fc_amd import _lib as L  # noqa: E402
from oracle import dflash_oracle as O  # noqa: E402
from workloads import configs, generate as G  # noqa: E402
from workloads.device import from_device, to_device  # noqa: E402

from gpu_harness import TOL, rel_l2, say  # noqa: E402


def _layer_and_caches(wl, prefill):
    lw = G.layer_weights(wl, 0)
    layer = L.Layer(*(to_device(lw[k], wl) for k in ("w_qkv", "w_o", "gamma_q", "gamma_k")),
                    n_h=wl.n_h, n_kv=wl.n_kv, d_h=wl.d_h, eps=wl.eps, rope_theta=wl.rope_theta)
    cap = (max(prefill) + 64 + wl.B + 63) // 64 * 64
    caches, K0, V0 = [], [], []
    for r in range(wl.R):
        k, v = G.prefill_kv(wl, 0, r, prefill[r])
        K0.append(k)
        V0.append(v)
    for _ in range(2):
        c = L.Cache(wl.R, wl.n_kv, wl.d_h, torch.bfloat16, cap, device="cuda")
        cu = np.concatenate([[0], np.cumsum(prefill)])
        kr = np.concatenate([k.transpose(1, 0, 2) for k in K0], axis=0)
        vr = np.concatenate([v.transpose(1, 0, 2) for v in V0], axis=0)
        L.dflash_cache_append(c, [int(x) for x in cu], to_device(kr, wl), to_device(vr, wl))
        caches.append(c)
    torch.cuda.synchronize()
    p = O.LayerParams(lw["w_qkv"], lw["w_o"], lw["gamma_q"], lw["gamma_k"], wl.n_h, wl.n_kv, wl.d_h, wl.eps,
                      wl.rope_theta, 0)
    return layer, caches, p, K0, V0


def test_noalloc_matches_workspace_call_twice():
    wl = configs.DECODE_8K.scaled(name="noalloc_gqa32x8_dh128_block16_bf16", d=1024, k_layers=2, R=2)
    prefill = [700, 1300]
    layer, (ca, cb), p, K, V = _layer_and_caches(wl, prefill)
    fc = G.fc_weights(wl)
    w_fc, g_h = to_device(fc["w_fc"], wl), to_device(fc["gamma_h"], wl)
    for call, n in enumerate([[9, 14], [3, 0]]):
        say(f"case noalloc call {call} n={n}")
        cu = [0, n[0], n[0] + n[1]]
        x, _, H = G.round_inputs(wl, call, n)
        T = cu[-1]
        C = torch.empty((max(T, 1), wl.d), dtype=torch.bfloat16, device="cuda")
        cws = torch.empty(max(L.dflash_ctx_project_ws_bytes(max(T, 1), wl.kd, wl.d, torch.bfloat16), 256),
                          dtype=torch.uint8, device="cuda")
        if T:
            L.dflash_ctx_project(to_device(x, wl), w_fc, g_h, wl.eps, C[:T], cws)
        Hd = to_device(H, wl)
        out_a = torch.full((wl.R * wl.B, wl.d), float("nan"), dtype=torch.bfloat16, device="cuda")
        out_b = out_a.clone()
        ws = torch.empty(L.dflash_kv_inject_attn_ws_bytes(layer, ca, T, wl.B), dtype=torch.uint8, device="cuda")
        L.dflash_kv_inject_attn(layer, ca, C[:T], cu, Hd, wl.B, out_a, ws)
        L.dflash_kv_inject_attn_noalloc(layer, cb, C[:T], cu, Hd, wl.B, out_b)
        torch.cuda.synchronize()
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), "outputs differ"
        assert ca.lengths() == cb.lengths()
        assert torch.equal(ca.k_pool.view(torch.int16), cb.k_pool.view(torch.int16))
        assert torch.equal(ca.v_pool.view(torch.int16), cb.v_pool.view(torch.int16))
        Cref = O.ctx_project(x, fc["w_fc"], fc["gamma_h"], wl.eps)
        got = from_device(out_b)
        for r in range(wl.R):
            res = O.kv_inject_layer(p, K[r], V[r], Cref[cu[r]:cu[r + 1]], H[r * wl.B:(r + 1) * wl.B])
            e = rel_l2(got[r * wl.B:(r + 1) * wl.B], res.out)
            assert e <= TOL["bf16"], f"call {call} seq {r}: rel-L2 {e:.3e}"
            K[r], V[r] = O.crop(res.K, res.V, K[r].shape[1] + n[r])
        keep = [prefill[r] + n[r] for r in range(wl.R)]
        for c in (ca, cb):
            L.dflash_cache_crop(c, keep)
        prefill = keep


def test_noalloc_refuses_calls_beyond_the_buffer():
    """16384 new context rows need over 64 MiB of q/k/v partial products: the
    call is refused (DFLASH_ERR_WORKSPACE) before anything is enqueued."""
    wl = configs.DECODE_8K.scaled(name="noalloc_too_big", R=1)
    layer, (ca, _), _, _, _ = _layer_and_caches(wl.scaled(name="noalloc_small_cache", d=wl.d), [64])
    T = 16384
    big = L.Cache(1, wl.n_kv, wl.d_h, torch.bfloat16, T + 128, device="cuda")
    C = torch.zeros((T, wl.d), dtype=torch.bfloat16, device="cuda")
    H = torch.zeros((wl.B, wl.d), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((wl.B, wl.d), dtype=torch.bfloat16, device="cuda")
    rc = L.LIB.dflash_kv_inject_attn_noalloc(L.C.byref(layer.desc), big.handle, C.data_ptr(), L._i32([0, T]),
                                             H.data_ptr(), wl.B, out.data_ptr(), None)
    torch.cuda.synchronize()
    assert rc == L.ERR_WORKSPACE
    assert big.lengths() == [0]
    assert int(out.view(torch.int16).abs().sum()) == 0
