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
            if wl.ring_capacity(li):
                self.caches.append(L.Cache(wl.R, wl.n_kv, wl.d_h, self.dtype, wl.ring_capacity(li), 0, 0, device,
                                           ring=True))
            elif wl.page_size:
                ps = wl.page_size
                pages = sum(-(-x // ps) for x in need) + wl.R
                maxp = max(-(-x // ps) for x in need) + 1
                self.caches.append(L.Cache(wl.R, wl.n_kv, wl.d_h, self.dtype, pages, ps, maxp, device))
            else:
                cap = _round_up(max(need), 64)
                self.caches.append(L.Cache(wl.R, wl.n_kv, wl.d_h, self.dtype, cap, 0, 0, device))
        max_T = int(sched.sum(axis=1).max()) if rounds else 0
        self.driver = DraftRound(self.w_fc, self.gamma_h, wl.eps, self.layers, self.caches, wl.B,
                                 max(max_T, 1), device)

    def prefill(self, kv_host):
        """kv_host[l][r] = (K, V) [n_kv, L_r, d_h] float32 storage values; appended
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
    """Seeded cache content before round 0, per layer and request."""
    L0 = G.prefill_lengths(wl)
    return [[G.prefill_kv(wl, li, r, int(L0[r])) for r in range(wl.R)] for li in range(wl.n_layers)]


def oracle_stack(wl, kv_host):
    fc = G.fc_weights(wl)
    layers = []
    for li in range(wl.n_layers):
        lw = G.layer_weights(wl, li)
        layers.append(O.LayerParams(lw["w_qkv"].astype(np.float64), lw["w_o"].astype(np.float64),
                                    lw["gamma_q"], lw["gamma_k"], wl.n_h, wl.n_kv, wl.d_h, wl.eps,
                                    wl.rope_theta, wl.layer_window(li)))
    K0 = [[kv_host[li][r][0] for r in range(wl.R)] for li in range(wl.n_layers)]
    V0 = [[kv_host[li][r][1] for r in range(wl.R)] for li in range(wl.n_layers)]
    return O.OracleStack(layers, fc["w_fc"].astype(np.float64), fc["gamma_h"], wl.eps, K0, V0)


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
