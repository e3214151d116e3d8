"""One draft round of a stack of KV-injection layers, as a sequence of C-ABI calls.

"DFlash KV Injection Walkthrough" Step 2 projects the new context rows once per
round and shares the result with every draft layer; Step 4 runs each layer on
the block rows; Step 7 and section 4 of "DFlash源码导读二 ..." cut every layer's
draft cache back to the accepted prefix (block start) afterwards.  Layers with
the residual flag chain H_{l+1} = H_l + o_proj_l through the library.  This
module only allocates device buffers and issues the library calls in that
order; all arithmetic runs in libdflash.so.
"""
from __future__ import annotations

import torch

from . import _lib as L


class DraftRound:
    def __init__(self, w_fc, gamma_h, eps, layers, caches, B, max_T, device="cuda"):
        assert len(layers) == len(caches) >= 1
        self.w_fc, self.gamma_h, self.eps = w_fc, gamma_h, float(eps)
        self.layers, self.caches, self.B = list(layers), list(caches), int(B)
        self.d = w_fc.shape[0]
        self.kd = w_fc.shape[1]
        self.dtype = w_fc.dtype
        R = caches[0].n_seqs
        self.C = torch.empty((max(max_T, 1), self.d), dtype=self.dtype, device=device)
        self.ctx_ws = torch.empty(max(L.dflash_ctx_project_ws_bytes(max_T, self.kd, self.d, self.dtype), 256),
                                  dtype=torch.uint8, device=device)
        ws = max(L.dflash_kv_inject_attn_ws_bytes(lay, c, max_T, B) for lay, c in zip(layers, caches))
        self.layer_ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)
        self.out = [torch.empty((R * B, self.d), dtype=self.dtype, device=device) for _ in layers]

    def run(self, x_raw, cu, H, stream=None):
        """x_raw [T, k*d] (request r at rows cu[r]..cu[r+1]-1), H [R*B, d].
        Returns every layer's output, [R*B, d] each; a residual layer's output
        is the next layer's block input."""
        T = int(cu[-1])
        C = self.C[:T]
        if T:
            L.dflash_ctx_project(x_raw, self.w_fc, self.gamma_h, self.eps, C, self.ctx_ws, stream)
        h = H
        for layer, cache, out in zip(self.layers, self.caches, self.out):
            before = cache.lengths()
            L.dflash_kv_inject_attn(layer, cache, C, cu, h, self.B, out, self.layer_ws, stream)
            L.dflash_cache_crop(cache, [before[r] + int(cu[r + 1] - cu[r]) for r in range(cache.n_seqs)], stream)
            h = out
        return self.out
