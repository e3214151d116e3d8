"""Set-up shared by the GPU parity tests: device copies of the seeded
workloads, caches prefilled through the C ABI, read-back of cache rows, and the
rel-L2 metric.  Marshalling only: the layer's arithmetic runs in libdflash.so on
the GPU side and in oracle/ on the reference side; this module computes
neither."""
from __future__ import annotations

import numpy as np
import torch

from block_diffusion_draft_fc_amd import _lib as L
from block_diffusion_draft_fc_amd.draft_round import DraftRound
from oracle import dflash_oracle as O
from workloads import generate as G
from workloads.device import from_device, to_device, torch_dtype

# rel-L2 bars: fp32 storage end to end, and bf16 storage with fp32 accumulation
TOL = {"f32": 1e-5, "bf16": 1e-2}


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def say(msg: str) -> None:
    print(msg, flush=True)


def _round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


class GpuModel:
    """Device weights, one cache per layer and a DraftRound driver for a workload."""

    def __init__(self, wl, rounds: int, device="cuda"):
        self.wl = wl
        self.dtype = torch_dtype(wl)
        fc = G.fc_weights(wl)
        self.w_fc = to_device(fc["w_fc"], wl, device)
        self.gamma_h = to_device(fc["gamma_h"], wl, device)
        self.L0 = G.prefill_lengths(wl)
        sched = G.schedule(wl)[:rounds]
        grow = sched.sum(axis=0) if rounds else np.zeros(wl.R, dtype=np.int64)
        self.layers, self.caches = [], []
        for li in range(wl.n_layers):
            lw = G.layer_weights(wl, li)
            self.layers.append(L.Layer(*(to_device(lw[k], wl, device) for k in ("w_qkv", "w_o", "gamma_q", "gamma_k")),
                                       n_h=wl.n_h, n_kv=wl.n_kv, d_h=wl.d_h, eps=wl.eps,
                                       rope_theta=wl.rope_theta, window=wl.layer_window(li),
                                       residual=wl.n_layers > 1))
            need = [int(self.L0[r] + grow[r] + wl.B) for r in range(wl.R)]
            cdt = torch.float8_e4m3fn if wl.kv_dtype == "fp8" else self.dtype
            sc = dict(k_scale=wl.k_scale, v_scale=wl.v_scale)
            if wl.ring_capacity(li):
                self.caches.append(L.Cache(wl.R, wl.n_kv, wl.d_h, cdt, wl.ring_capacity(li), 0, 0, device,
                                           ring=True, **sc))
            elif wl.page_size:
                ps = wl.page_size
                pages = sum(-(-x // ps) for x in need) + wl.R
                maxp = max(-(-x // ps) for x in need) + 1
                self.caches.append(L.Cache(wl.R, wl.n_kv, wl.d_h, cdt, pages, ps, maxp, device, **sc))
            else:
                cap = _round_up(max(need), 64)
                self.caches.append(L.Cache(wl.R, wl.n_kv, wl.d_h, cdt, cap, 0, 0, device, **sc))
        max_T = int(sched.sum(axis=1).max()) if rounds else 0
        self.driver = DraftRound(self.w_fc, self.gamma_h, wl.eps, self.layers, self.caches, wl.B,
                                 max(max_T, 1), device)

    def prefill(self, kv_host):
        """kv_host[l][r] = (K, V) [n_kv, L_r, d_h] float32 storage values (uint8
        E4M3 codes for fp8 caches); appended
        through dflash_cache_append (one call per layer and all requests; a ring
        takes them in calls of at most its capacity rows per request)."""
        for li, cache in enumerate(self.caches):
            step = cache.capacity if cache.ring else max([kv_host[li][r][0].shape[1] for r in range(self.wl.R)] + [1])
            longest = max(kv_host[li][r][0].shape[1] for r in range(self.wl.R))
            for a in range(0, longest, step):
                ks, vs, cu = [], [], [0]
                for r in range(self.wl.R):
                    k, v = kv_host[li][r]
                    ks.append(np.ascontiguousarray(k[:, a:a + step].transpose(1, 0, 2)))
                    vs.append(np.ascontiguousarray(v[:, a:a + step].transpose(1, 0, 2)))
                    cu.append(cu[-1] + ks[-1].shape[0])
                if cu[-1] == 0:
                    continue
                if cache.fp8:
                    kd = torch.from_numpy(np.concatenate(ks, axis=0)).to("cuda")
                    vd = torch.from_numpy(np.concatenate(vs, axis=0)).to("cuda")
                else:
                    kd = to_device(np.concatenate(ks, axis=0), self.wl)
                    vd = to_device(np.concatenate(vs, axis=0), self.wl)
                L.dflash_cache_append(cache, cu, kd, vd)
        torch.cuda.synchronize()

    def round(self, x_raw, cu, H):
        xd = to_device(x_raw, self.wl) if x_raw.shape[0] else torch.empty((0, self.wl.kd), dtype=self.dtype,
                                                                           device="cuda")
        outs = self.driver.run(xd, [int(c) for c in cu], to_device(H, self.wl))
        torch.cuda.synchronize()
        return [from_device(o) for o in outs]


def prefill_host(wl):
    """Seeded cache content before round 0, per layer and request (E4M3 codes
    for fp8 caches)."""
    L0 = G.prefill_lengths(wl)
    draw = G.prefill_kv_fp8 if wl.kv_dtype == "fp8" else G.prefill_kv
    return [[draw(wl, li, r, int(L0[r])) for r in range(wl.R)] for li in range(wl.n_layers)]


def kv_values(wl, k, v):
    """The values a cache holds for stored rows (codes times the scales for
    fp8 caches, else the stored values)."""
    if wl.kv_dtype == "fp8":
        return O.e4m3_decode(k) * wl.k_scale, O.e4m3_decode(v) * wl.v_scale
    return k, v


def check_fp8_codes(got, exact, scale, what):
    """Codes an fp8 cache holds for layer-written rows against the oracle's
    values before storage.  The GPU quantises values computed from its bf16
    context rows C: each element of C is off by up to 2^-9 of itself, so a
    projected element x_j = sum_i C_i W_ji is off by about 2^-9 / sqrt(3) of the
    RMS of x (1.13e-3 RMS, one standard deviation; the per-head norm of K
    keeps that ratio).  Let t = 8e-3 RMS (7 standard deviations).  A code that
    is the nearest E4M3 code of some x' within t of x = exact / scale lies
    within |nearest(x) - x| + 2 t of x, which is what every code must meet;
    at most 10% of codes may differ from nearest(x) (about 4% expected for
    N(0, 1) rows).  Returns the count of such codes."""
    got = np.asarray(got).astype(np.uint8)
    x = np.asarray(exact, dtype=np.float64) / scale
    want = O.e4m3_encode(x)
    a, b = O.e4m3_decode(got), O.e4m3_decode(want)
    bad = a != b                       # +0 and -0 are the same value
    if not bad.any():
        return 0
    t = 8e-3 * float(np.sqrt(np.mean(x * x)))
    ok = np.abs(a[bad] - x[bad]) <= np.abs(b[bad] - x[bad]) + 2 * t
    assert np.all(ok), f"{what}: {int((~ok).sum())} of {bad.size} codes off the nearest value"
    assert bad.mean() <= 0.10, f"{what}: {int(bad.sum())} codes of {bad.size} not the nearest"
    return int(bad.sum())


def oracle_stack(wl, kv_host):
    fc = G.fc_weights(wl)
    layers = []
    for li in range(wl.n_layers):
        lw = G.layer_weights(wl, li)
        layers.append(O.LayerParams(lw["w_qkv"].astype(np.float64), lw["w_o"].astype(np.float64),
                                    lw["gamma_q"], lw["gamma_k"], wl.n_h, wl.n_kv, wl.d_h, wl.eps,
                                    wl.rope_theta, wl.layer_window(li)))
    K0 = [[kv_values(wl, *kv_host[li][r])[0] for r in range(wl.R)] for li in range(wl.n_layers)]
    V0 = [[kv_values(wl, *kv_host[li][r])[1] for r in range(wl.R)] for li in range(wl.n_layers)]
    scales = (wl.k_scale, wl.v_scale) if wl.kv_dtype == "fp8" else None
    return O.OracleStack(layers, fc["w_fc"].astype(np.float64), fc["gamma_h"], wl.eps, K0, V0, scales)


def v_rows_view(vp):
    """V pool tiles [..., n_kv, tiles, d_h, 64] (slot j's head dim i in tile
    j // 64, row i, column j % 64) as rows [n_kv, tiles * 64, d_h] (any leading
    dims are folded into the row axis after n_kv)."""
    if vp.dim() == 4:
        g, t, d, w = vp.shape
        return vp.permute(0, 1, 3, 2).reshape(g, t * w, d)
    g, p, t, d, w = vp.shape
    return vp.permute(0, 1, 2, 4, 3).reshape(g, p * t * w, d)


def ring_rows(cache: L.Cache, s: int, lo: int):
    """Rows of positions lo .. len-1 of sequence s of a ring cache (slot
    pos % capacity) read back as float64: K, V [n_kv, len - lo, d_h]."""
    n = cache.lengths()[s]
    slots = torch.tensor([p % cache.capacity for p in range(lo, n)], dtype=torch.long,
                         device=cache.k_pool.device)
    K = cache.k_pool[s][:, slots, :]
    V = v_rows_view(cache.v_pool[s])[:, slots, :]
    return from_device(K.contiguous()), from_device(V.contiguous())


def cache_rows(cache: L.Cache, s: int):
    """Logical rows of sequence s read back from the device pools as float64:
    K, V [n_kv, len, d_h]."""
    assert not cache.ring, "a ring holds only its last rows: use ring_rows"
    n = cache.lengths()[s]
    if cache.page_size == 0:
        K = cache.k_pool[s, :, :n, :]
        V = v_rows_view(cache.v_pool[s])[:, :n, :]
    else:
        ps = cache.page_size
        pages = cache.block_table()[s][: -(-n // ps)]
        idx = torch.tensor(pages, dtype=torch.long, device=cache.k_pool.device)
        K = cache.k_pool[idx].permute(1, 0, 2, 3).reshape(cache.n_kv, -1, cache.d_h)[:, :n]
        V = v_rows_view(cache.v_pool[idx].transpose(0, 1))[:, :n]
    return from_device(K.contiguous()), from_device(V.contiguous())
