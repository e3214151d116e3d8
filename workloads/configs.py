"""Workload definitions for the DFlash KV-injection attention layer.

Each workload fixes the layer shapes, the batch (requests R, block size B),
the cache state a round starts from and how many rounds run.  The shapes follow
the walkthrough example (DFlash KV Injection Walkthrough, "example setup" table:
d = 512, 8 heads of 64, three target layers, block of 4, a 3-token prompt) and
Qwen3-4B / Qwen3-8B-shaped draft layers.  Nothing here computes any part of the
method; the module only names sizes and seeds.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    d: int                 # hidden size
    n_h: int               # query heads
    n_kv: int              # key/value heads
    d_h: int               # head dim (explicit, may differ from d / n_h)
    k_layers: int          # number of target layers concatenated into the raw context
    B: int                 # block size (1 anchor + B-1 mask rows)
    R: int                 # requests per round
    rounds: int            # draft rounds
    dtype: str             # "f32" or "bf16" storage (fp32 accumulation everywhere)
    seed: int
    # cache state at the start of round 0
    prefill: str = "none"          # "none" | "fixed" | "uniform"
    prefill_len: int = 0           # "fixed": every request starts at this length
    prefill_range: Tuple[int, int] = (0, 0)   # "uniform": inclusive range per request
    # newly accepted context rows per request and round
    n_new: str = "fixed"           # "fixed" | "uniform"
    n_fixed: int = 0               # "fixed": rows in round 0 (the only round)
    n_range: Tuple[int, int] = (1, 16)        # "uniform": inclusive range
    # block rows: "iid" = every row N(0,1); "anchor_mask" = row 0 a fresh anchor,
    # rows 1.. one shared mask vector fixed per seed
    block_rows: str = "anchor_mask"
    # cache layout
    page_size: int = 0             # 0 = contiguous per request; else paged
    # layer stack: number of layers and which are sliding-window layers
    n_layers: int = 1
    window: int = 0                # sliding window of the sliding layers (0 = none)
    sliding_layers: Tuple[int, ...] = ()
    # sliding layers keep a bounded ring cache (window + B - 1 rows, rounded up
    # to 64, at least the rows of one round) instead of the whole context
    ring: bool = False
    eps: float = 1e-6
    rope_theta: float = 1e6
    # cache element type: "same" as the layer, or "fp8" (E4M3 bytes read as
    # value * k_scale / v_scale; bf16 layers only)
    kv_dtype: str = "same"
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def kd(self) -> int:
        return self.k_layers * self.d

    @property
    def group(self) -> int:
        return self.n_h // self.n_kv

    def layer_window(self, layer: int) -> int:
        return self.window if layer in self.sliding_layers else 0

    def ring_capacity(self, layer: int) -> int:
        """Rows of the layer's ring cache, 0 for an unbounded cache."""
        if not (self.ring and layer in self.sliding_layers):
            return 0
        n_max = self.n_fixed if self.n_new == "fixed" else self.n_range[1]
        need = max(self.window + self.B - 1, n_max + self.B)
        return (need + 63) // 64 * 64

    def scaled(self, **kw) -> "Workload":
        """A copy with some fields replaced (smaller parity cases)."""
        return replace(self, **kw)


# Walkthrough-sized layer: d 512, MHA 8 x 64, target layers 3/7/11 -> 1536-wide
# raw context, 3 prompt positions (0-2), block of 4 (positions 3-6), fp32, no cache.
WALKTHROUGH = Workload(
    name="walkthrough_d512_mha8x64_ctx3_block4_f32",
    d=512, n_h=8, n_kv=8, d_h=64, k_layers=3, B=4, R=1, rounds=1, dtype="f32",
    seed=0, prefill="none", n_new="fixed", n_fixed=3, block_rows="iid")

# Qwen3-4B-shaped layer on a fresh 1024-row context plus one block of 16.
FRESH_CTX = Workload(
    name="fresh_ctx1024_d2560_gqa32x8_dh128_block16_bf16",
    d=2560, n_h=32, n_kv=8, d_h=128, k_layers=5, B=16, R=1, rounds=1, dtype="bf16",
    seed=1, prefill="none", n_new="fixed", n_fixed=1024)

# Qwen3-8B-shaped layer in steady-state decode: cache pre-filled to 8192 rows,
# 64 rounds, each appending 1..16 accepted context rows plus a block of 16.
DECODE_8K = Workload(
    name="decode_ctx8k_d4096_gqa32x8_dh128_block16_bf16",
    d=4096, n_h=32, n_kv=8, d_h=128, k_layers=5, B=16, R=1, rounds=64, dtype="bf16",
    seed=2, prefill="fixed", prefill_len=8192, n_new="uniform", n_range=(1, 16))

# 16 ragged requests, contexts uniform on 512..16384, paged cache of 256-row pages.
RAGGED_PAGED = Workload(
    name="ragged16_ctx512-16k_paged256_d4096_gqa32x8_block16_bf16",
    d=4096, n_h=32, n_kv=8, d_h=128, k_layers=5, B=16, R=16, rounds=64, dtype="bf16",
    seed=3, prefill="uniform", prefill_range=(512, 16384), n_new="uniform",
    n_range=(1, 16), page_size=256)

# Five-layer hybrid stack: sliding-window layers (window 4096) alternate with
# full-attention layers, batch 4, 32768-row contexts, 32 rounds.
STACK5_HYBRID = Workload(
    name="stack5_hybrid_swa4096_ctx32k_batch4_d4096_gqa32x8_block16_bf16",
    d=4096, n_h=32, n_kv=8, d_h=128, k_layers=5, B=16, R=4, rounds=32, dtype="bf16",
    seed=4, prefill="fixed", prefill_len=32768, n_new="uniform", n_range=(1, 16),
    n_layers=5, window=4096, sliding_layers=(0, 2, 4))

ALL = (WALKTHROUGH, FRESH_CTX, DECODE_8K, RAGGED_PAGED, STACK5_HYBRID)

# Vocabulary of the Qwen3 family's lm_head (the draft head of a Qwen3-8B-shaped
# draft model reads the target's lm_head: [151936, 4096]).
QWEN3_VOCAB = 151936
BY_NAME = {w.name: w for w in ALL}
