"""Plain fp64 CPU oracle for the DFlash KV-injection attention layer.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.  The GPU library never calls it, and it
imports nothing from the GPU package: the two share no code.

Sources (cited by page title and section):
  [W]  "DFlash KV Injection Walkthrough": Step 2 (projection and norm),
       Step 4.1-4.5 (Q projection, dual-stream K/V, RoPE alignment, attention,
       output projection), Step 6-7 (acceptance, state update).
  [S]  "DFlash源码导读二 Qwen3DFlashAttention注意力实现全解析": section 1 (QKV
       projection, QK-RMSNorm, head_dim, GQA groups), 2 (dual-stream K/V),
       3 (RoPE window), 4 (KV cache update and crop), 5 (sliding window), and the
       non-causal key design.
  [T]  "KV Cache + Speculative Decoding 面试 Cheat Sheet": section 4.2 and 6.3
       (GQA: each K/V head serves a contiguous group of query heads), 2.1 and
       4.5 (a cache element stored in one byte as fp8).

Everything is float64.  Inputs arrive as float32 arrays holding exact bf16 or
fp32 values and are upcast without any rounding afterwards.  Library routines
used as steps: numpy matmul, sqrt, exp, cos, sin.

Readings taken where the pages leave a step open (the numbers refer to the list
of readings kept with the design notes):
  R2  W_fc is stored [d, k*d] (output x input); a context row is raw_row . W_fc^T.
  R3  RMSNorm(x) = x / sqrt(mean(x^2) + eps) * gamma over the normalised axis
      (d for hidden_norm, d_h for the per-head Q/K norms, gains shared by heads).
  R4  no biases in q/k/v/o projections.
  R5  RoPE pairs element i with i + d_h/2 (rotate_half), w_i = theta^(-2i/d_h).
  R6  the RoPE window of a round covers positions [L, L + n + B); cached keys keep
      the rotation they got when appended.
  R7  block rows are appended too, then the caller crops to L + n.
  R10 query head h reads K/V head h // (n_h / n_kv).
  R12 sliding layers: key j is visible to query i iff pos_i - pos_j < window
      (no upper bound: still non-causal inside the block).
  R14 layer stacks chain H_{l+1} = H_l + out_l (the decoder MLP is not on the
      pages, so the chaining is a builder choice); every layer reads the one
      context C of the round and keeps its own cache, cropped after the round.
  R23 an fp8 cache element is an OCP FP8 E4M3 byte: code = the nearest E4M3
      value of x / scale (ties to the even mantissa, magnitudes from 448 up
      saturated to 448), read back as value(code) * scale, with one fp32
      scale for K and one for V per cache; nothing else changes precision.
  R21 the draft head samples greedily: the token of a row is the first index of
      its maximal logit (temperature sampling would need random draws the
      pages do not fix).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# norms and the context projection
# --------------------------------------------------------------------------

def rms_norm(x, gamma, eps: float) -> np.ndarray:
    """RMSNorm over the last axis (reading R3).  [W] Step 2 names hidden_norm as
    an RMSNorm over d; [S] section 1 names the per-head q_norm/k_norm over d_h."""
    x = f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * f64(gamma)


def ctx_project(x_raw, w_fc, gamma_h, eps: float) -> np.ndarray:
    """Context C = hidden_norm(fc(raw)), [W] Step 2.

    x_raw [T, k*d]: each row is the k target-layer vectors of one position,
    concatenated in layer order ([W] Step 1).  w_fc is stored [d, k*d]
    (reading R2: only raw_row . W_fc^T is dimensionally consistent with the
    stated 1536 x 512 shape).  fc has no bias."""
    u = f64(x_raw) @ f64(w_fc).T
    return rms_norm(u, gamma_h, eps)


# --------------------------------------------------------------------------
# rotary position embedding
# --------------------------------------------------------------------------

def rope_inv_freq(d_h: int, theta: float) -> np.ndarray:
    """w_i = theta^(-2i/d_h), i < d_h/2 (reading R5)."""
    i = np.arange(d_h // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / d_h)


def rope(x, positions, theta: float) -> np.ndarray:
    """Rotate rows of x [..., P, d_h] by their positions [P], [W] Step 4.3.

    rotate_half pairing: the first half and the second half of a head vector
    form the pairs, x' = x*cos + rotate_half(x)*sin with rotate_half(x) =
    [-x_hi, x_lo] and cos/sin repeated over both halves."""
    x = f64(x)
    d_h = x.shape[-1]
    half = d_h // 2
    ang = f64(positions)[:, None] * rope_inv_freq(d_h, theta)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


# --------------------------------------------------------------------------
# the layer
# --------------------------------------------------------------------------

@dataclass
class LayerParams:
    """One KV-injection attention layer.  w_qkv rows are W_Q | W_K | W_V, each
    block stored output x input; w_o is [d, n_h*d_h]."""
    w_qkv: np.ndarray
    w_o: np.ndarray
    gamma_q: np.ndarray
    gamma_k: np.ndarray
    n_h: int
    n_kv: int
    d_h: int
    eps: float = 1e-6
    theta: float = 1e6
    window: int = 0

    def split(self):
        qd, kvd = self.n_h * self.d_h, self.n_kv * self.d_h
        w = f64(self.w_qkv)
        return w[:qd], w[qd:qd + kvd], w[qd + kvd:qd + 2 * kvd]


def project_q(p: LayerParams, H) -> np.ndarray:
    """Q = QNorm(H W_Q), viewed per head: [n_h, B, d_h] (not yet rotated).
    [W] Step 4.1: queries come from the block stream only."""
    wq, _, _ = p.split()
    B = H.shape[0]
    q = (f64(H) @ wq.T).reshape(B, p.n_h, p.d_h)
    q = rms_norm(q, p.gamma_q, p.eps)
    return q.transpose(1, 0, 2)


def project_kv(p: LayerParams, C, H):
    """Dual-stream K/V, [W] Step 4.2 and [S] section 2: the same k_proj and
    v_proj act on the context rows C and on the block rows H; the results are
    concatenated along the sequence, context first.  K gets the per-head norm,
    V does not.  Returns k [n_kv, n+B, d_h] (normed, not rotated), v alike."""
    _, wk, wv = p.split()
    S = np.concatenate([f64(C), f64(H)], axis=0)
    rows = S.shape[0]
    k = rms_norm((S @ wk.T).reshape(rows, p.n_kv, p.d_h), p.gamma_k, p.eps)
    v = (S @ wv.T).reshape(rows, p.n_kv, p.d_h)
    return k.transpose(1, 0, 2), v.transpose(1, 0, 2)


def visible(qpos, kpos, window: int) -> np.ndarray:
    """[B, L_tot] bool: which keys each query may attend to.  Full layers see
    every key ([W] Step 4.4: no causal mask; [S] key design: is_causal False and
    no attention mask).  Sliding layers (reading R12) see keys with
    pos_q - pos_k < window."""
    qpos, kpos = np.asarray(qpos), np.asarray(kpos)
    if window <= 0:
        return np.ones((qpos.size, kpos.size), dtype=bool)
    return (qpos[:, None] - kpos[None, :]) < window


def gqa_attention(q, K, V, qpos, kpos, window: int = 0):
    """Softmax attention of rotated queries q [n_h, B, d_h] over the cache
    K, V [n_kv, L_tot, d_h], [W] Step 4.4: A = softmax(q'.k'^T / sqrt(d_h)),
    out = A V, scale d_h^-0.5.  Query head h reads K/V head h // (n_h/n_kv)
    ([S] section 1, [T] 6.3 repeat_interleave).
    Returns o [n_h, B, d_h] and the weights A [n_h, B, L_tot]."""
    q, K, V = f64(q), f64(K), f64(V)
    n_h, B, d_h = q.shape
    n_kv, L_tot, _ = K.shape
    group = n_h // n_kv
    scale = d_h ** -0.5
    vis = visible(qpos, kpos, window)
    o = np.empty((n_h, B, d_h))
    A = np.empty((n_h, B, L_tot))
    for h in range(n_h):
        g = h // group
        s = (q[h] @ K[g].T) * scale
        s = np.where(vis, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        a = e / e.sum(axis=1, keepdims=True)
        A[h] = a
        o[h] = a @ V[g]
    return o, A


def o_proj(o, w_o) -> np.ndarray:
    """[W] Step 4.5: heads concatenated per row (head h at columns h*d_h ..),
    then one projection back to d.  Only block rows produce output."""
    o = f64(o)
    n_h, B, d_h = o.shape
    return o.transpose(1, 0, 2).reshape(B, n_h * d_h) @ f64(w_o).T


@dataclass
class LayerResult:
    out: np.ndarray        # [B, d]
    K: np.ndarray          # cache after the append, [n_kv, L + n + B, d_h]
    V: np.ndarray
    q: np.ndarray          # rotated queries [n_h, B, d_h]
    weights: np.ndarray    # attention weights [n_h, B, L + n + B]
    qpos: np.ndarray
    kpos: np.ndarray
    k_exact: np.ndarray = None   # appended rows before fp8 storage [n_kv, n + B, d_h]
    v_exact: np.ndarray = None


def kv_inject_layer(p: LayerParams, K_cache, V_cache, C, H, kv_scales=None) -> LayerResult:
    """One request through one layer, [W] Step 4 with the cache of [S] section 4.

    K_cache, V_cache [n_kv, L, d_h] hold rotated keys and raw values of
    positions 0..L-1.  C [n, d] are this round's new context rows and H [B, d]
    the block rows.  The RoPE window covers positions L .. L+n+B-1 (reading R6,
    [S] section 3): keys take all of it (context rows then block rows), queries
    the last B positions ([W] Step 4.3).  The rotated keys and raw values of
    all n + B rows are appended (reading R7) before attention, which runs over
    every cached key.

    kv_scales = (k_scale, v_scale) stores the cache in fp8 (reading R23): the
    appended rows become e4m3_quantize(k, k_scale) and e4m3_quantize(v,
    v_scale) before attention reads them, like every cached row (K_cache and
    V_cache then hold such values already)."""
    K_cache, V_cache = f64(K_cache), f64(V_cache)
    L = K_cache.shape[1]
    n, B = C.shape[0], H.shape[0]
    pos = L + np.arange(n + B, dtype=np.int64)
    qpos = pos[n:]
    q = rope(project_q(p, H), qpos, p.theta)
    k, v = project_kv(p, C, H)
    k = rope(k, pos, p.theta)
    k_exact, v_exact = k, v
    if kv_scales is not None:
        k = e4m3_quantize(k, kv_scales[0])
        v = e4m3_quantize(v, kv_scales[1])
    K = np.concatenate([K_cache, k], axis=1)
    V = np.concatenate([V_cache, v], axis=1)
    kpos = np.arange(L + n + B, dtype=np.int64)
    o, A = gqa_attention(q, K, V, qpos, kpos, p.window)
    return LayerResult(o_proj(o, p.w_o), K, V, q, A, qpos, kpos, k_exact, v_exact)


def crop(K, V, new_len: int):
    """Keep the accepted prefix, [S] section 4 and [W] Step 7: the draft cache
    is cut back to the block start, dropping block rows and rejected rows."""
    if not 0 <= new_len <= K.shape[1]:
        raise ValueError("crop beyond the current length")
    return K[:, :new_len], V[:, :new_len]


# --------------------------------------------------------------------------
# draft head, [W] Step 5
# --------------------------------------------------------------------------

def draft_head(h, gamma_f, eps: float, w_lm, B: int):
    """[W] Step 5: after the last draft layer and a final RMSNorm over d, the
    last B-1 rows of every request's block (the first row holds the known
    token, whose prediction is dropped) go through lm_head (w_lm [vocab, d],
    output x input, no bias), and greedy sampling (reading R21) keeps each
    row's argmax.  h [R*B, d].  Returns logits [R*(B-1), vocab] and token ids
    [R*(B-1)]; row r*(B-1)+j is block position j+1 of request r."""
    h = f64(h)
    R = h.shape[0] // B
    x = rms_norm(h, gamma_f, eps).reshape(R, B, -1)[:, 1:, :].reshape(R * (B - 1), -1)
    logits = x @ f64(w_lm).T
    return logits, np.argmax(logits, axis=-1)


# --------------------------------------------------------------------------
# round bookkeeping, [W] Step 6 and Step 7
# --------------------------------------------------------------------------

def acceptance_length(draft_tail, posterior_head) -> int:
    """Number of leading draft tokens the target agrees with: the cumulative
    product of per-position matches, summed."""
    m = np.asarray([a == b for a, b in zip(draft_tail, posterior_head)], dtype=np.int64)
    return int(np.cumprod(m).sum())


def next_start(start: int, acc: int) -> int:
    """The accepted tokens plus the target's own correction advance the start."""
    return start + acc + 1


def new_context_rows(acc: int) -> int:
    """Rows of new context injected next round: the accepted positions plus the
    corrected one."""
    return acc + 1


def accept_round(draft_ids, posterior):
    """[W] Step 6 and Step 7 for a batch of R requests.  draft_ids [R, B-1]:
    the draft tokens of block positions 1..B-1; posterior [R, B]: the target's
    prediction of the token after each block position 0..B-1.  Per request the
    draft token of position j+1 is checked against the target's prediction
    from position j (block_output_ids[:, 1:] against posterior[:, :-1]);
    acc counts the leading matches.  The next round injects new_context_rows
    (acc) context rows, and its block opens with the target's own token at
    the first position not accepted, posterior[acc] (the correction that
    replaces the rejected draft token).  Returns (acc, next_rows, anchor),
    int64 arrays of length R."""
    draft_ids = np.asarray(draft_ids).reshape(len(posterior), -1)
    posterior = np.asarray(posterior)
    R = posterior.shape[0]
    acc = np.zeros(R, dtype=np.int64)
    rows = np.zeros(R, dtype=np.int64)
    anchor = np.zeros(R, dtype=np.int64)
    for r in range(R):
        acc[r] = acceptance_length(list(draft_ids[r]), list(posterior[r][:-1]))
        rows[r] = new_context_rows(int(acc[r]))
        anchor[r] = posterior[r][acc[r]]
    return acc, rows, anchor


# --------------------------------------------------------------------------
# fp8 cache elements, [T] sections 2.1 and 4.5 (one byte per element), in the
# OCP FP8 E4M3 format (reading R23)
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 byte: bit 7 the sign, bits 6..3 the exponent field e
    (bias 7), bits 2..0 the mantissa m.  e = 0 holds the subnormals
    (m / 8) * 2^-6; any other e holds (1 + m / 8) * 2^(e - 7), except that
    e = 15 with m = 7 is NaN.  No infinities; the largest finite magnitude is
    1.75 * 2^8 = 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e, m = (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def e4m3_encode(x) -> np.ndarray:
    """The E4M3 byte nearest each value, ties to the even mantissa (reading
    R23).  Magnitudes of 448 and more saturate to 448; NaN becomes 0x7F; the
    sign of zero is kept.

    A magnitude a in the binade [2^e, 2^(e+1)) (e >= -6; the subnormals share
    the spacing of e = -6) lies on the grid of steps 2^(e-3): q = a * 2^(3-e),
    rounded to an integer ties-to-even, is 8 + m for a normal value and m for
    a subnormal one, so the magnitude bits are (e + 6) * 8 + q; q = 16 carries
    into the next binade with m = 0, which the same formula gives."""
    x = f64(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, k = np.frexp(a)
    e = np.where(a < 2.0 ** -6, -6, k - 1)
    q = np.rint(np.where(np.isnan(a), 0.0, a) * np.exp2(3.0 - e))
    bits = (e + 6) * 8 + q.astype(np.int64)
    bits = np.where(np.signbit(x), bits | 0x80, bits)
    bits = np.where(np.isnan(x), 0x7F, bits)
    return bits.astype(np.uint8)


def e4m3_quantize(x, scale: float) -> np.ndarray:
    """What an fp8 cache holds for x: value(code(x / scale)) * scale."""
    return e4m3_decode(e4m3_encode(f64(x) / scale)) * scale


# --------------------------------------------------------------------------
# multi-request rounds and layer stacks
# --------------------------------------------------------------------------

class OracleStack:
    """Per-layer, per-request caches for a batch of R requests through a stack
    of layers.  One round: C = ctx_project(new raw rows) once, shared by every
    layer ([W] Step 2: one context for all draft layers); then each layer runs
    kv_inject_layer per request, chaining H_{l+1} = H_l + out_l (reading R14);
    then every layer's cache is cropped to L + n."""

    def __init__(self, layers, w_fc, gamma_h, eps, K0, V0, kv_scales=None):
        """K0[l][r], V0[l][r]: [n_kv, L_r, d_h] cache content before round 0.
        kv_scales = (k_scale, v_scale): fp8 caches (reading R23), whose
        content K0, V0 already holds fp8 values times the scales."""
        self.layers = list(layers)
        self.w_fc, self.gamma_h, self.eps = w_fc, gamma_h, eps
        self.kv_scales = kv_scales
        self.K = [[f64(k) for k in row] for row in K0]
        self.V = [[f64(v) for v in row] for row in V0]
        # fp8 caches: the values of the cached rows before storage (the given
        # rows for K0, V0), to tell where a rounding decision was close
        self.Kx = [[k.copy() for k in row] for row in self.K] if kv_scales else None
        self.Vx = [[v.copy() for v in row] for row in self.V] if kv_scales else None

    def lengths(self, layer: int = 0):
        return [k.shape[1] for k in self.K[layer]]

    def round(self, x_raw, cu, H, B: int):
        """x_raw [T, k*d] with request r at rows cu[r]..cu[r+1]-1; H [R*B, d].
        Returns outputs [n_layers][R*B, d] (each layer's o_proj output) and the
        last layer's LayerResult per request."""
        R = len(cu) - 1
        C = ctx_project(x_raw, self.w_fc, self.gamma_h, self.eps)
        h = f64(H).copy()
        outs, last = [], []
        for li, p in enumerate(self.layers):
            out_l = np.empty_like(h)
            res_l = []
            for r in range(R):
                L = self.K[li][r].shape[1]
                res = kv_inject_layer(p, self.K[li][r], self.V[li][r],
                                      C[cu[r]:cu[r + 1]], h[r * B:(r + 1) * B], self.kv_scales)
                out_l[r * B:(r + 1) * B] = res.out
                n = cu[r + 1] - cu[r]
                self.K[li][r], self.V[li][r] = crop(res.K, res.V, L + n)
                if self.kv_scales:
                    self.Kx[li][r], self.Vx[li][r] = crop(np.concatenate([self.Kx[li][r], res.k_exact], axis=1),
                                                          np.concatenate([self.Vx[li][r], res.v_exact], axis=1),
                                                          L + n)
                res_l.append(res)
            outs.append(out_l)
            last = res_l
            h = h + out_l
        return outs, last
