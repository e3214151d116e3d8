"""Integer model of the draft KV cache: lengths, pages, free list, pool bytes.

TEST INFRASTRUCTURE (same import rule as dflash_oracle).  It is the bit-exact
reference for the library's cache append and crop: it moves payload words
without arithmetic, so every byte of the pools, every length and every page
table entry can be compared for equality.

Semantics follow "DFlash源码导读二 Qwen3DFlashAttention注意力实现全解析"
section 4 (the cache receives the new rows of a round and is later cut back to
the accepted prefix) and "DFlash KV Injection Walkthrough" Step 7 (the cache
grows round by round by the accepted positions).  The paged layout follows
"KV Cache + Speculative Decoding 面试 Cheat Sheet" sections 5.2-5.3 and 6.2
(fixed-size pages from a global pool, one page table per request mapping
logical page -> physical page, pages returned to a free list).  Prefix sharing
and copy-on-write are not modelled (no request shares pages here).

Pool layout (as declared in the library header):
  contiguous (page_size == 0), capacity = rows per sequence:
      K pool [n_seqs][n_kv][capacity][d_h]
      V pool [n_seqs][n_kv][capacity / 64][d_h][64]
  paged (page_size > 0), capacity = pages in the pool:
      K pool [capacity][n_kv][page_size][d_h]
      V pool [capacity][n_kv][page_size / 64][d_h][64]
  V is stored transposed in tiles of 64 slots: slot j's head dim i sits in
  tile j // 64, row i, column j % 64.  (The library takes capacities and page
  sizes in multiples of 64; for the small sizes of the logic tests the model
  pads its last tile.)
  Row `pos` of sequence s lives in logical page pos // page_size, slot
  pos % page_size.  Allocation takes the lowest-numbered free page; sequences
  are served in index order and each sequence's new logical pages in order.
  Crop returns every page at or beyond ceil(new_len / page_size).

Ring (contiguous only): the bounded cache of a sliding-window layer, the
rotating cache that "DFlash源码导读二 Qwen3DFlashAttention注意力实现全解析"
(the MLX comparison table) pairs with the trim of the full cache.  Row `pos`
lives in slot pos % capacity and lengths may exceed the capacity; with hw the
highest position ever written plus one, the rows at positions
[max(0, hw - capacity), len) are held.  One append brings at most `capacity`
rows per sequence.  A layer call with window W, n new context rows and B
block rows reads keys from max(0, len + n - W + 1) on; it needs W > 0,
W + B - 1 <= capacity, n + B <= capacity, and that first key still held.
"""
from __future__ import annotations

import numpy as np

OK, ERR_ARG, ERR_SHAPE, ERR_DTYPE, ERR_RANGE, ERR_CAPACITY = 0, -1, -2, -3, -4, -5
V_TILE = 64   # slots per transposed V tile


class CacheError(Exception):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


class CacheModel:
    def __init__(self, n_seqs, n_kv, d_h, page_size, capacity, max_pages_per_seq=0,
                 word=np.uint16, ring=False):
        self.n_seqs, self.n_kv, self.d_h = int(n_seqs), int(n_kv), int(d_h)
        self.page_size, self.capacity = int(page_size), int(capacity)
        self.max_pages = int(max_pages_per_seq)
        self.word = word
        self.ring = bool(ring)
        if self.ring and self.page_size:
            raise CacheError(ERR_SHAPE, "a ring is a contiguous cache")
        self.len = [0] * self.n_seqs
        self.hw = [0] * self.n_seqs
        if self.paged:
            self.K = np.zeros((capacity, n_kv, page_size, d_h), dtype=word)
            self.V = np.zeros((capacity, n_kv, -(-page_size // V_TILE), d_h, V_TILE), dtype=word)
            self.pages = [[] for _ in range(self.n_seqs)]
            self.free = set(range(self.capacity))
        else:
            self.K = np.zeros((n_seqs, n_kv, capacity, d_h), dtype=word)
            self.V = np.zeros((n_seqs, n_kv, -(-capacity // V_TILE), d_h, V_TILE), dtype=word)

    @property
    def paged(self) -> bool:
        return self.page_size > 0

    def _pages_for(self, n_rows: int) -> int:
        return -(-n_rows // self.page_size)

    def append(self, cu_rows, k_rows, v_rows):
        """Rows [cu[s], cu[s+1]) of k_rows / v_rows [n_rows, n_kv, d_h] go to
        positions len_s .. len_s + n_s - 1.  All checks run before any change."""
        cu = [int(c) for c in cu_rows]
        if len(cu) != self.n_seqs + 1 or cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])):
            raise CacheError(ERR_ARG, "cu_rows must be non-decreasing from 0")
        n = [cu[s + 1] - cu[s] for s in range(self.n_seqs)]
        if self.paged:
            need = 0
            for s in range(self.n_seqs):
                want = self._pages_for(self.len[s] + n[s])
                if want > self.max_pages:
                    raise CacheError(ERR_CAPACITY, "sequence exceeds max_pages_per_seq")
                need += max(0, want - len(self.pages[s]))
            if need > len(self.free):
                raise CacheError(ERR_CAPACITY, "page pool exhausted")
            for s in range(self.n_seqs):
                want = self._pages_for(self.len[s] + n[s])
                while len(self.pages[s]) < want:
                    pg = min(self.free)
                    self.free.remove(pg)
                    self.pages[s].append(pg)
        else:
            for s in range(self.n_seqs):
                if self.ring and n[s] > self.capacity:
                    raise CacheError(ERR_CAPACITY, "more rows than ring slots in one call")
                if not self.ring and self.len[s] + n[s] > self.capacity:
                    raise CacheError(ERR_CAPACITY, "sequence exceeds capacity")
        for s in range(self.n_seqs):
            for j in range(n[s]):
                pos = self.len[s] + j
                krow, vrow = k_rows[cu[s] + j], v_rows[cu[s] + j]
                if self.paged:
                    pg, slot = self.pages[s][pos // self.page_size], pos % self.page_size
                    self.K[pg, :, slot, :] = krow
                    self.V[pg, :, slot // V_TILE, :, slot % V_TILE] = vrow
                else:
                    slot = pos % self.capacity
                    self.K[s, :, slot, :] = krow
                    self.V[s, :, slot // V_TILE, :, slot % V_TILE] = vrow
            self.len[s] += n[s]
            self.hw[s] = max(self.hw[s], self.len[s])

    def crop(self, new_len):
        new_len = [int(x) for x in new_len]
        if len(new_len) != self.n_seqs:
            raise CacheError(ERR_ARG, "one length per sequence")
        for s in range(self.n_seqs):
            if not 0 <= new_len[s] <= self.len[s]:
                raise CacheError(ERR_RANGE, "crop beyond the current length")
        for s in range(self.n_seqs):
            self.len[s] = new_len[s]
            if self.paged:
                keep = self._pages_for(new_len[s])
                for pg in self.pages[s][keep:]:
                    self.free.add(pg)
                del self.pages[s][keep:]

    def layer_call_status(self, n, B: int, window: int) -> int:
        """Status of a layer call on a ring with n[s] new context rows, B block
        rows and the given window (checked before anything changes)."""
        if window <= 0:
            return ERR_SHAPE
        if window + B - 1 > self.capacity:
            return ERR_CAPACITY
        for s in range(self.n_seqs):
            if max(0, self.len[s] + int(n[s]) - window + 1) < self.hw[s] - self.capacity:
                return ERR_RANGE
        for s in range(self.n_seqs):
            if int(n[s]) + B > self.capacity:
                return ERR_CAPACITY
        return OK

    def held(self, s: int):
        """Ring: (lo, K, V) with K, V [n_kv, len - lo, d_h] the rows of positions
        lo .. len - 1 that the ring still holds, lo = max(0, hw - capacity)."""
        lo = max(0, self.hw[s] - self.capacity)
        L = self.len[s]
        K = np.empty((self.n_kv, max(0, L - lo), self.d_h), dtype=self.word)
        V = np.empty((self.n_kv, max(0, L - lo), self.d_h), dtype=self.word)
        for pos in range(lo, L):
            slot = pos % self.capacity
            K[:, pos - lo, :] = self.K[s, :, slot, :]
            V[:, pos - lo, :] = self.V[s, :, slot // V_TILE, :, slot % V_TILE]
        return lo, K, V

    def block_table(self):
        return [list(p) for p in self.pages] if self.paged else None

    def pages_in_use(self) -> int:
        return sum(len(p) for p in self.pages) if self.paged else 0

    def rows(self, s: int):
        """Logical view of sequence s: K, V as [n_kv, len, d_h] words (not for
        rings, which hold only the last rows: see `held`)."""
        if self.ring:
            raise ValueError("a ring holds only its last rows")
        L = self.len[s]
        K = np.empty((self.n_kv, L, self.d_h), dtype=self.word)
        V = np.empty((self.n_kv, L, self.d_h), dtype=self.word)
        for pos in range(L):
            if self.paged:
                pg, slot = self.pages[s][pos // self.page_size], pos % self.page_size
                K[:, pos, :] = self.K[pg, :, slot, :]
                V[:, pos, :] = self.V[pg, :, slot // V_TILE, :, slot % V_TILE]
            else:
                K[:, pos, :] = self.K[s, :, pos, :]
                V[:, pos, :] = self.V[s, :, pos // V_TILE, :, pos % V_TILE]
        return K, V
