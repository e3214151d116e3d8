"""Seeded synthetic inputs for the DFlash KV-injection attention workloads.

This module only draws numbers.  It holds none of the method's arithmetic, so
both the fp64 oracle and the GPU path may use it.

Every tensor comes back as a float32 numpy array.  For bf16 workloads the
values are already rounded to bf16 (round to nearest, ties to even), so the same
array gives the GPU its exact storage bits (`bf16_bits`) and the oracle its exact
values (`.astype(np.float64)`).

Value distributions (workload descriptions): raw context rows, anchor and mask
rows ~ N(0, 1); weights ~ N(0, 1/fan_in) with fan_in the input width; RMSNorm
gains 1 + N(0, 0.1^2).  The cache a round starts from is itself an input of the
round; rows present before round 0 are drawn K ~ N(0, 1), V ~ N(0, 1), the
statistics of QK-normed keys and of values projected from a normed context.

Each draw has its own counter-addressed stream, np.random.default_rng over
SeedSequence([seed, tag, i, j, ...]), so any piece can be regenerated alone and
in any order.
"""
from __future__ import annotations

import numpy as np

from .configs import Workload

# stream tags
(_FC, _LAYER, _PREFILL_KV, _PREFILL_LEN, _SCHED, _RAW, _ANCHOR, _MASK, _H_IID, _HEAD, _HEAD_IN,
 _ACCEPT, _PREFILL_FP8) = range(1, 14)


def _rng(seed: int, *tags: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), *map(int, tags)]))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 holding the nearest bf16 value (ties to even).

    Inputs are finite, so no NaN/Inf special case is needed."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are exactly bf16 (storage bits)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (b >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x: np.ndarray, wl: Workload) -> np.ndarray:
    x = x.astype(np.float32, copy=False)
    return round_to_bf16(x) if wl.dtype == "bf16" else x


def _normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def fc_weights(wl: Workload):
    """W_fc stored [d, k*d] (output x input, row-major) and the hidden_norm gain [d]."""
    g = _rng(wl.seed, _FC)
    w_fc = _normal(g, (wl.d, wl.kd), 1.0 / np.sqrt(wl.kd))
    gamma_h = 1.0 + _normal(g, (wl.d,), 0.1)
    return {"w_fc": _store(w_fc, wl), "gamma_h": _store(gamma_h, wl)}


def layer_weights(wl: Workload, layer: int = 0):
    """One layer: w_qkv [(n_h + 2 n_kv) d_h, d] with rows W_Q | W_K | W_V,
    w_o [d, n_h d_h], q/k norm gains [d_h]."""
    g = _rng(wl.seed, _LAYER, layer)
    qd, kvd = wl.n_h * wl.d_h, wl.n_kv * wl.d_h
    w_qkv = _normal(g, (qd + 2 * kvd, wl.d), 1.0 / np.sqrt(wl.d))
    w_o = _normal(g, (wl.d, qd), 1.0 / np.sqrt(qd))
    gamma_q = 1.0 + _normal(g, (wl.d_h,), 0.1)
    gamma_k = 1.0 + _normal(g, (wl.d_h,), 0.1)
    return {"w_qkv": _store(w_qkv, wl), "w_o": _store(w_o, wl),
            "gamma_q": _store(gamma_q, wl), "gamma_k": _store(gamma_k, wl)}


def prefill_lengths(wl: Workload) -> np.ndarray:
    """Cache length of every request at the start of round 0."""
    if wl.prefill == "none":
        return np.zeros(wl.R, dtype=np.int64)
    if wl.prefill == "fixed":
        return np.full(wl.R, wl.prefill_len, dtype=np.int64)
    lo, hi = wl.prefill_range
    return _rng(wl.seed, _PREFILL_LEN).integers(lo, hi + 1, size=wl.R).astype(np.int64)


def prefill_kv(wl: Workload, layer: int, r: int, L: int):
    """Cache rows of request r, layer `layer`, at positions 0..L-1 before round 0.
    Returns K, V as [n_kv, L, d_h] (post-RoPE K, raw V)."""
    g = _rng(wl.seed, _PREFILL_KV, layer, r)
    k = _normal(g, (wl.n_kv, L, wl.d_h))
    v = _normal(g, (wl.n_kv, L, wl.d_h))
    return _store(k, wl), _store(v, wl)


def prefill_kv_fp8(wl: Workload, layer: int, r: int, L: int):
    """Cache rows of request r before round 0 for an fp8 cache, drawn directly
    as E4M3 bytes (no arithmetic on them here): sign bit and 3 mantissa bits
    uniform, exponent field uniform over 4..8, i.e. magnitudes 1/8 .. 3.75
    before the cache's scale.  Returns uint8 K, V codes [n_kv, L, d_h]."""
    g = _rng(wl.seed, _PREFILL_FP8, layer, r)

    def codes():
        sign = g.integers(0, 2, size=(wl.n_kv, L, wl.d_h)) << 7
        expo = g.integers(4, 9, size=(wl.n_kv, L, wl.d_h)) << 3
        mant = g.integers(0, 8, size=(wl.n_kv, L, wl.d_h))
        return (sign | expo | mant).astype(np.uint8)
    return codes(), codes()


def schedule(wl: Workload) -> np.ndarray:
    """n[round, r]: newly accepted context rows per request and round."""
    if wl.n_new == "fixed":
        return np.full((wl.rounds, wl.R), wl.n_fixed, dtype=np.int64)
    lo, hi = wl.n_range
    return _rng(wl.seed, _SCHED).integers(lo, hi + 1, size=(wl.rounds, wl.R)).astype(np.int64)


def mask_row(wl: Workload) -> np.ndarray:
    """The one mask-token embedding shared by every block's rows 1..B-1."""
    return _store(_normal(_rng(wl.seed, _MASK), (wl.d,)), wl)


def raw_rows(wl: Workload, rnd: int, r: int, n: int) -> np.ndarray:
    """Raw context rows [n, k*d] of request r in round rnd (k layer vectors per row)."""
    return _store(_normal(_rng(wl.seed, _RAW, rnd, r), (n, wl.kd)), wl)


def block_rows(wl: Workload, rnd: int, r: int) -> np.ndarray:
    """Block stream H [B, d] of request r in round rnd."""
    if wl.block_rows == "iid":
        return _store(_normal(_rng(wl.seed, _H_IID, rnd, r), (wl.B, wl.d)), wl)
    h = np.empty((wl.B, wl.d), dtype=np.float32)
    h[0] = _store(_normal(_rng(wl.seed, _ANCHOR, rnd, r), (wl.d,)), wl)
    h[1:] = mask_row(wl)[None, :]
    return h


def round_inputs(wl: Workload, rnd: int, n_per_req):
    """All requests of one round, packed: X_raw [T, k*d] with request r's rows at
    [cu[r], cu[r+1]), H [R*B, d] with request r's block at rows r*B .. r*B+B-1."""
    n_per_req = [int(x) for x in n_per_req]
    cu = np.zeros(wl.R + 1, dtype=np.int64)
    cu[1:] = np.cumsum(n_per_req)
    x = np.empty((int(cu[-1]), wl.kd), dtype=np.float32)
    h = np.empty((wl.R * wl.B, wl.d), dtype=np.float32)
    for r in range(wl.R):
        x[cu[r]:cu[r + 1]] = raw_rows(wl, rnd, r, n_per_req[r])
        h[r * wl.B:(r + 1) * wl.B] = block_rows(wl, rnd, r)
    return x, cu, h


def head_weights(wl: Workload, vocab: int):
    """Draft head: the final-norm gain [d] and lm_head [vocab, d] (output x
    input), drawn like every other weight (N(0, 1/d), gain 1 + N(0, 0.1^2))."""
    g = _rng(wl.seed, _HEAD, vocab)
    gamma_f = 1.0 + _normal(g, (wl.d,), 0.1)
    w_lm = _normal(g, (vocab, wl.d), 1.0 / np.sqrt(wl.d))
    return {"gamma_f": _store(gamma_f, wl), "w_lm": _store(w_lm, wl)}


def head_input(wl: Workload, rnd: int = 0) -> np.ndarray:
    """Rows [R*B, d] that the draft head reads (the stack's output for the
    blocks), N(0, 1)."""
    return _store(_normal(_rng(wl.seed, _HEAD_IN, rnd), (wl.R * wl.B, wl.d)), wl)


def accept_tokens(seed: int, R: int, B: int, vocab: int, rnd: int = 0):
    """Token ids for the acceptance of a round: posterior [R, B] uniform on
    [0, vocab), and draft [R, B-1] that agrees with posterior[r][:-1] on a
    planted prefix of k_r positions (k_r uniform on 0..B-1, the spread of
    acceptance lengths 1..B of the decode workloads), differs at position k_r
    and is uniform after it (later positions may agree again).
    Returns (draft int32 [R, B-1], posterior int32 [R, B], k int64 [R])."""
    g = _rng(seed, _ACCEPT, R, B, rnd)
    post = g.integers(0, vocab, size=(R, B), dtype=np.int64)
    k = g.integers(0, B, size=R, dtype=np.int64)
    draft = g.integers(0, vocab, size=(R, max(B - 1, 0)), dtype=np.int64)
    for r in range(R):
        draft[r, :k[r]] = post[r, :k[r]]
        if k[r] < B - 1:
            draft[r, k[r]] = (post[r, k[r]] + 1 + g.integers(0, vocab - 1)) % vocab
    return draft.astype(np.int32), post.astype(np.int32), k
