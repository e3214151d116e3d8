"""Pins for the fp64 oracle, checked against what the pages and the mathematics
fix rather than against the oracle itself.

Sources: "DFlash KV Injection Walkthrough" (shapes of Steps 1-4, the scaling
0.125, RoPE relative-position identity of Step 4.3, non-causal 4 x 7 attention
of Step 4.4, acceptance example of Step 6, cache growth of Step 7);
"DFlash源码导读二 Qwen3DFlashAttention注意力实现全解析" (same k_proj/v_proj on both
streams, GQA groups); "KV Cache + Speculative Decoding 面试 Cheat Sheet" 6.3
(grouped attention equals attention with repeat_interleave'd K/V heads).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dflash_oracle as O
from workloads import configs, generate as G

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "walkthrough.json")))


def _params(wl, layer=0):
    lw = G.layer_weights(wl, layer)
    return O.LayerParams(lw["w_qkv"], lw["w_o"], lw["gamma_q"], lw["gamma_k"],
                         wl.n_h, wl.n_kv, wl.d_h, wl.eps, wl.rope_theta, wl.layer_window(layer))


def _tiny_params(rng, d=8, n_h=4, n_kv=2, d_h=4, window=0, theta=1e4):
    qd, kvd = n_h * d_h, n_kv * d_h
    return O.LayerParams(rng.standard_normal((qd + 2 * kvd, d)) / math.sqrt(d),
                         rng.standard_normal((d, qd)) / math.sqrt(qd),
                         1 + 0.1 * rng.standard_normal(d_h), 1 + 0.1 * rng.standard_normal(d_h),
                         n_h, n_kv, d_h, 1e-6, theta, window)


# ---------------------------------------------------------------- walkthrough

def test_walkthrough_shapes_and_positions():
    wl = configs.WALKTHROUGH
    s, sh = GOLDEN["setup"], GOLDEN["shapes"]
    assert (wl.d, wl.n_h, wl.d_h, wl.k_layers, wl.B) == (s["d"], s["n_h"], s["d_h"], s["k"], s["block_size"])
    assert wl.d_h == wl.d // wl.n_h
    fc = G.fc_weights(wl)
    x, cu, H = G.round_inputs(wl, 0, [wl.n_fixed])
    assert list(x.shape) == sh["target_hidden_raw"]
    assert list(fc["w_fc"].T.shape) == sh["w_fc_math"]
    C = O.ctx_project(x, fc["w_fc"], fc["gamma_h"], wl.eps)
    assert list(C.shape) == sh["C"] and list(H.shape) == sh["H"]
    p = _params(wl)
    K0 = np.zeros((wl.n_kv, 0, wl.d_h))
    res = O.kv_inject_layer(p, K0, K0, C, H)
    assert list(res.q.shape) == sh["Q"]
    assert list(res.K.shape) == sh["K"] and list(res.V.shape) == sh["V"]
    assert list(res.weights.shape[1:]) == sh["A"]
    assert list(res.out.shape) == sh["attn_out"]
    pos = GOLDEN["positions"]
    assert list(res.qpos) == pos["q"] and list(res.kpos) == pos["k"]
    # the cos/sin table covers the whole window, one row per position, width d_h
    assert [len(pos["window"]), wl.d_h] == sh["cos_sin"]


def test_scaling_is_printed_value():
    """Two keys with score gap g: the first weight is 1/(1+exp(-g*scale)), the
    scale printed for d_h = 64 being 0.125."""
    d_h = GOLDEN["scaling"]["d_h"]
    scale = GOLDEN["scaling"]["value"]
    q = np.zeros((1, 1, d_h)); q[0, 0, 0] = 3.0
    K = np.zeros((1, 2, d_h)); K[0, 0, 0] = 2.0; K[0, 1, 0] = -1.0
    V = np.zeros((1, 2, d_h)); V[0, 0, 1] = 1.0
    _, A = O.gqa_attention(q, K, V, [0], [0, 0])
    gap = 3.0 * 2.0 - 3.0 * (-1.0)
    assert abs(A[0, 0, 0] - 1.0 / (1.0 + math.exp(-gap * scale))) < 1e-15


def test_softmax_rows_sum_to_one_and_no_causal_mask():
    wl = configs.WALKTHROUGH
    fc = G.fc_weights(wl)
    x, _, H = G.round_inputs(wl, 0, [wl.n_fixed])
    C = O.ctx_project(x, fc["w_fc"], fc["gamma_h"], wl.eps)
    K0 = np.zeros((wl.n_kv, 0, wl.d_h))
    res = O.kv_inject_layer(_params(wl), K0, K0, C, H)
    assert np.max(np.abs(res.weights.sum(axis=-1) - 1.0)) < 1e-12
    # every query sees every key, including later block positions
    assert np.all(res.weights > 0)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 33)) * rng.uniform(0.01, 10, size=(7, 1))
    eps = 1e-3
    y = O.rms_norm(x, np.ones(33), eps)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-12)
    # scale invariance as eps -> 0, and the gain multiplies elementwise
    g = rng.uniform(0.5, 1.5, 33)
    assert np.allclose(O.rms_norm(5.0 * x, g, 0.0), O.rms_norm(x, g, 0.0), rtol=1e-12)
    assert np.allclose(O.rms_norm(x, g, 0.0), O.rms_norm(x, np.ones(33), 0.0) * g, rtol=1e-12)


def test_ctx_project_brute_force():
    rng = np.random.default_rng(6)
    T, kd, d = 3, 6, 4
    x, w, g = rng.standard_normal((T, kd)), rng.standard_normal((d, kd)), rng.standard_normal(d)
    C = O.ctx_project(x, w, g, 1e-6)
    for t in range(T):
        u = [sum(x[t, i] * w[o, i] for i in range(kd)) for o in range(d)]
        r = math.sqrt(sum(v * v for v in u) / d + 1e-6)
        for o in range(d):
            assert abs(C[t, o] - u[o] / r * g[o]) < 1e-12


# ---------------------------------------------------------------- RoPE

def test_rope_equals_complex_rotation():
    """rotate_half pairs (x_i, x_{i+d/2}) rotate like the complex number
    x_i + j x_{i+d/2} multiplied by exp(j p w_i)."""
    rng = np.random.default_rng(7)
    d_h, theta = 16, 1e6
    x = rng.standard_normal((5, d_h))
    pos = np.array([0, 1, 7, 8191, 33000])
    y = O.rope(x, pos, theta)
    half = d_h // 2
    for r in range(5):
        for i in range(half):
            w = theta ** (-2.0 * i / d_h)
            z = complex(x[r, i], x[r, i + half]) * complex(math.cos(pos[r] * w), math.sin(pos[r] * w))
            assert abs(y[r, i] - z.real) < 1e-12 and abs(y[r, i + half] - z.imag) < 1e-12


def test_rope_group_properties():
    rng = np.random.default_rng(8)
    d_h = 128
    x = rng.standard_normal((4, d_h))
    p = np.array([0, 3, 100, 9000]); q = np.array([5, 2, 77, 24000])
    assert np.allclose(O.rope(x, np.zeros(4), 1e6), x, atol=0)
    assert np.allclose(np.linalg.norm(O.rope(x, p, 1e6), axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.allclose(O.rope(O.rope(x, p, 1e6), q, 1e6), O.rope(x, p + q, 1e6), atol=1e-10)


@pytest.mark.parametrize("delta", [1, 37, 8192, 100000])
def test_rope_relative_position_invariance(delta):
    """q'_i . k'_j depends on j - i only: shifting every position by delta
    leaves all scores unchanged (Step 4.3)."""
    rng = np.random.default_rng(9)
    d_h = 64
    q, k = rng.standard_normal((4, d_h)), rng.standard_normal((7, d_h))
    qpos, kpos = np.arange(3, 7), np.arange(7)
    s0 = O.rope(q, qpos, 1e6) @ O.rope(k, kpos, 1e6).T
    s1 = O.rope(q, qpos + delta, 1e6) @ O.rope(k, kpos + delta, 1e6).T
    assert np.max(np.abs(s1 - s0)) <= 1e-9 * np.max(np.abs(s0))


def test_rope_example_pair_and_wrong_offset():
    """The walkthrough's example: the query at position 5 against the key at
    position 2 sees a relative rotation of -3; the wrong window (queries at
    0..3) would put that query at position 2, relative rotation 0."""
    ex = GOLDEN["positions"]["example_pair"]
    rng = np.random.default_rng(10)
    d_h = 64
    q, k = rng.standard_normal(d_h), rng.standard_normal(d_h)
    s = O.rope(q[None], np.array([ex["q_pos"]]), 1e6) @ O.rope(k[None], np.array([ex["k_pos"]]), 1e6).T
    rel = O.rope(k[None], np.array([ex["relative"]]), 1e6)
    assert abs(s[0, 0] - (q @ rel[0])) < 1e-12
    wrong = O.rope(q[None], np.array([ex["wrong_q_pos"]]), 1e6) @ O.rope(k[None], np.array([ex["k_pos"]]), 1e6).T
    assert abs(wrong[0, 0] - q @ O.rope(k[None], np.array([ex["wrong_relative"]]), 1e6)[0]) < 1e-12
    assert abs(wrong[0, 0] - s[0, 0]) > 1e-3


def test_layer_tail_offset_matters():
    """Queries on the last B window positions (correct) versus on the first B
    (the wrong reading): outputs must differ by far more than any tolerance."""
    wl = configs.WALKTHROUGH
    p = _params(wl)
    fc = G.fc_weights(wl)
    x, _, H = G.round_inputs(wl, 0, [wl.n_fixed])
    C = O.ctx_project(x, fc["w_fc"], fc["gamma_h"], wl.eps)
    K0 = np.zeros((wl.n_kv, 0, wl.d_h))
    good = O.kv_inject_layer(p, K0, K0, C, H)
    q_wrong = O.rope(O.project_q(p, H), np.arange(wl.B), p.theta)
    o, _ = O.gqa_attention(q_wrong, good.K, good.V, np.arange(wl.B), good.kpos)
    bad = O.o_proj(o, p.w_o)
    rel = np.linalg.norm(bad - good.out) / np.linalg.norm(good.out)
    assert rel > 1e-2


# ---------------------------------------------------------------- attention

def test_gqa_equals_repeated_kv_mha():
    rng = np.random.default_rng(11)
    n_h, n_kv, B, L, d_h = 8, 2, 3, 11, 16
    q = rng.standard_normal((n_h, B, d_h))
    K, V = rng.standard_normal((n_kv, L, d_h)), rng.standard_normal((n_kv, L, d_h))
    o_g, _ = O.gqa_attention(q, K, V, np.arange(B), np.arange(L))
    Kr, Vr = np.repeat(K, n_h // n_kv, axis=0), np.repeat(V, n_h // n_kv, axis=0)
    o_m, _ = O.gqa_attention(q, Kr, Vr, np.arange(B), np.arange(L))
    assert np.max(np.abs(o_g - o_m)) < 1e-12


def test_position_zero_reduces_to_library_sdpa():
    """All positions 0: RoPE is the identity and attention is textbook SDPA,
    here torch's CPU scaled_dot_product_attention in float64."""
    rng = np.random.default_rng(12)
    n_h, n_kv, B, L, d_h = 8, 2, 5, 9, 32
    q = rng.standard_normal((n_h, B, d_h))
    K, V = rng.standard_normal((n_kv, L, d_h)), rng.standard_normal((n_kv, L, d_h))
    qr = O.rope(q, np.zeros(B), 1e6)
    Kr = O.rope(K, np.zeros(L), 1e6)
    o, _ = O.gqa_attention(qr, Kr, V, np.zeros(B, int), np.zeros(L, int))
    tq = torch.from_numpy(q)[None]
    tk = torch.from_numpy(K).repeat_interleave(n_h // n_kv, dim=0)[None]
    tv = torch.from_numpy(V).repeat_interleave(n_h // n_kv, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=False)[0].numpy()
    assert np.max(np.abs(o - ref)) < 1e-12


def test_single_key_closed_form():
    """No cache, no context, one block row: attention over the row's own key
    returns its own value, so out = v_own . W_O^T with v_own repeated per group."""
    rng = np.random.default_rng(13)
    p = _tiny_params(rng)
    d = p.w_qkv.shape[1]
    H = rng.standard_normal((1, d))
    res = O.kv_inject_layer(p, np.zeros((p.n_kv, 0, p.d_h)), np.zeros((p.n_kv, 0, p.d_h)),
                            np.zeros((0, d)), H)
    wv = p.w_qkv[(p.n_h + p.n_kv) * p.d_h:]
    v = (H @ wv.T).reshape(p.n_kv, p.d_h)
    attn = np.concatenate([v[h // (p.n_h // p.n_kv)] for h in range(p.n_h)])
    assert np.allclose(res.out[0], attn @ p.w_o.T, atol=1e-12)


def test_dual_stream_rows_are_independent():
    """The same k_proj/v_proj act on the context and the block rows: the
    context rows of the cache do not depend on the block, and after the crop
    the cache equals what the context alone produces."""
    rng = np.random.default_rng(14)
    p = _tiny_params(rng)
    d = p.w_qkv.shape[1]
    L, n, B = 3, 2, 3
    K0, V0 = rng.standard_normal((p.n_kv, L, p.d_h)), rng.standard_normal((p.n_kv, L, p.d_h))
    C = rng.standard_normal((n, d))
    r1 = O.kv_inject_layer(p, K0, V0, C, rng.standard_normal((B, d)))
    r2 = O.kv_inject_layer(p, K0, V0, C, rng.standard_normal((B, d)))
    k1, v1 = O.crop(r1.K, r1.V, L + n)
    k2, v2 = O.crop(r2.K, r2.V, L + n)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    k_ctx, v_ctx = O.project_kv(p, C, np.zeros((0, d)))
    assert np.allclose(k1[:, L:], O.rope(k_ctx, L + np.arange(n), p.theta), atol=1e-13)
    assert np.allclose(v1[:, L:], v_ctx, atol=1e-13)


# ---------------------------------------------------------------- window

def test_window_closed_forms():
    rng = np.random.default_rng(15)
    L, n, B = 5, 2, 3
    p_full = _tiny_params(rng)
    K0, V0 = rng.standard_normal((p_full.n_kv, L, p_full.d_h)), rng.standard_normal((p_full.n_kv, L, p_full.d_h))
    d = p_full.w_qkv.shape[1]
    C, H = rng.standard_normal((n, d)), rng.standard_normal((B, d))
    full = O.kv_inject_layer(p_full, K0, V0, C, H)
    for W in (L + n + B, L + n + B + 100):
        p_w = O.LayerParams(**{**p_full.__dict__, "window": W})
        assert np.array_equal(O.kv_inject_layer(p_w, K0, V0, C, H).out, full.out)
    p1 = O.LayerParams(**{**p_full.__dict__, "window": 1})
    r1 = O.kv_inject_layer(p1, K0, V0, C, H)
    for b in range(B):
        qp = L + n + b
        seen = set(np.nonzero(r1.weights[0, b] > 0)[0].tolist())
        assert seen == set(range(qp, L + n + B))   # itself and the later block rows


# ---------------------------------------------------------------- brute force

def _brute_layer(p, K0, V0, C, H, quant_k=None, quant_v=None):
    """Scalar-loop formulation: explicit 2x2 rotations, explicit exp and sums,
    K/V heads repeated explicitly for every query head.  quant_k / quant_v map
    an appended row to what the cache stores (identity when None)."""
    quant_k = quant_k or (lambda r: r)
    quant_v = quant_v or (lambda r: r)
    d_h, n_h, n_kv = p.d_h, p.n_h, p.n_kv
    half = d_h // 2
    W = p.w_qkv
    rows = [list(r) for r in C] + [list(r) for r in H]
    n, B, L = len(C), len(H), K0.shape[1]

    def lin(x, first_row, count):
        return [sum(x[i] * W[first_row + o][i] for i in range(len(x))) for o in range(count)]

    def norm(v, g):
        ms = sum(t * t for t in v) / len(v)
        return [v[i] / math.sqrt(ms + p.eps) * g[i] for i in range(len(v))]

    def rot(v, pos):
        out = [0.0] * d_h
        for i in range(half):
            a = pos * p.theta ** (-2.0 * i / d_h)
            m = [[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]]
            out[i] = m[0][0] * v[i] + m[0][1] * v[i + half]
            out[i + half] = m[1][0] * v[i] + m[1][1] * v[i + half]
        return out

    Kc = [[list(K0[g, j]) for j in range(L)] for g in range(n_kv)]
    Vc = [[list(V0[g, j]) for j in range(L)] for g in range(n_kv)]
    for t, x in enumerate(rows):
        kx = lin(x, n_h * d_h, n_kv * d_h)
        vx = lin(x, (n_h + n_kv) * d_h, n_kv * d_h)
        for g in range(n_kv):
            Kc[g].append(quant_k(rot(norm(kx[g * d_h:(g + 1) * d_h], p.gamma_k), L + t)))
            Vc[g].append(quant_v(vx[g * d_h:(g + 1) * d_h]))
    Kh = [Kc[h * n_kv // n_h] for h in range(n_h)]     # explicit repetition per query head
    Vh = [Vc[h * n_kv // n_h] for h in range(n_h)]
    out = []
    for b in range(B):
        qx = lin(list(H[b]), 0, n_h * d_h)
        qpos = L + n + b
        concat = []
        for h in range(n_h):
            qh = rot(norm(qx[h * d_h:(h + 1) * d_h], p.gamma_q), qpos)
            keys = [j for j in range(L + n + B) if p.window <= 0 or qpos - j < p.window]
            sc = [sum(qh[i] * Kh[h][j][i] for i in range(d_h)) / math.sqrt(d_h) for j in keys]
            mx = max(sc)
            ex = [math.exp(s - mx) for s in sc]
            tot = sum(ex)
            concat += [sum(ex[a] / tot * Vh[h][j][i] for a, j in enumerate(keys)) for i in range(d_h)]
        out.append([sum(concat[i] * p.w_o[o][i] for i in range(len(concat))) for o in range(len(p.w_o))])
    return np.array(out), Kc, Vc


@pytest.mark.parametrize("L,n,B,window", [(0, 0, 1, 0), (0, 3, 2, 0), (5, 1, 3, 0), (2, 2, 2, 0),
                                          (4, 3, 3, 3), (5, 2, 1, 1), (3, 0, 3, 2)])
def test_brute_force_tiny(L, n, B, window):
    rng = np.random.default_rng(100 + 7 * L + 3 * n + B)
    p = _tiny_params(rng, window=window)
    d = p.w_qkv.shape[1]
    K0, V0 = rng.standard_normal((p.n_kv, L, p.d_h)), rng.standard_normal((p.n_kv, L, p.d_h))
    C, H = rng.standard_normal((n, d)), rng.standard_normal((B, d))
    res = O.kv_inject_layer(p, K0, V0, C, H)
    out, Kc, Vc = _brute_layer(p, K0, V0, C, H)
    assert np.max(np.abs(res.out - out)) < 1e-12
    assert np.max(np.abs(res.K - np.array(Kc))) < 1e-12
    assert np.max(np.abs(res.V - np.array(Vc))) < 1e-12


# ---------------------------------------------------------------- fp8 cache elements
# "KV Cache + Speculative Decoding 面试 Cheat Sheet" 2.1 and 4.5 give one byte
# per fp8 element; the format is OCP FP8 E4M3 (sign, 4 exponent bits with bias
# 7, 3 mantissa bits, no infinities, S.1111.111 = NaN, largest value 448).

def _e4m3_grid():
    """The 127 non-negative finite E4M3 magnitudes in code order, listed from
    the format's definition: 8 subnormal steps of 2^-9, then 8 steps per binade
    from 2^-6 up to 1.75 * 2^8."""
    sub = [m * 2.0 ** -9 for m in range(8)]
    norm = [(8 + m) * 2.0 ** (e - 10) for e in range(1, 16) for m in range(8)][:-1]
    return np.array(sub + norm)


def _brute_e4m3(x):
    """Nearest grid magnitude by exhaustive search; a tie goes to the even code
    (codes count up with the magnitude, so the even index); saturation at
    448; the sign is re-applied.  Returns the code."""
    grid = _e4m3_grid()
    a = min(abs(x), 448.0)
    dist = np.abs(grid - a)
    best = np.flatnonzero(dist == dist.min())
    code = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
    return code | (0x80 if math.copysign(1.0, x) < 0 else 0)


def test_e4m3_format_values():
    """Codes whose values the format fixes: zero, the smallest subnormal, the
    largest subnormal, the smallest normal, one and its neighbours, the largest
    value, NaN, and the negative codes mirroring the positive ones."""
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x37: 0.9375,
             0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0x7D: 416.0, 0x80: -0.0,
             0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}
    for c, v in table.items():
        assert O.e4m3_decode(np.uint8(c)) == v, hex(c)
    assert math.copysign(1.0, O.e4m3_decode(np.uint8(0x80))) == -1.0
    assert np.isnan(O.e4m3_decode(np.uint8(0x7F))) and np.isnan(O.e4m3_decode(np.uint8(0xFF)))
    vals = O.e4m3_decode(np.arange(127, dtype=np.uint8))
    assert np.array_equal(vals, _e4m3_grid())          # codes 0..126 in order of magnitude
    assert np.array_equal(O.e4m3_decode(np.arange(128, 255, dtype=np.uint8)), -vals)


def test_e4m3_matches_library_cast():
    """Every code decodes as torch.float8_e4m3fn does, and in-range values
    encode as its round-to-nearest-even cast does (the library saturates
    nothing, so out-of-range values are pinned separately)."""
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ours = O.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(ours[ok], lib[ok]) and np.array_equal(np.signbit(ours[ok]), np.signbit(lib[ok]))
    rng = np.random.default_rng(23)
    x = rng.standard_normal(200000) * np.exp2(rng.uniform(-13.0, 9.0, 200000))
    x = x[np.abs(x) < 448.0]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), want)


def test_e4m3_encode_brute_force_and_ties():
    """Exhaustive nearest search on random magnitudes, on every midpoint
    between neighbouring codes (ties to the even code) and just beside each;
    every finite code round-trips; saturation and NaN."""
    grid = _e4m3_grid()
    mids = (grid[:-1] + grid[1:]) / 2
    rng = np.random.default_rng(5)
    xs = list(mids) + list(np.nextafter(mids, 0)) + list(np.nextafter(mids, 1e9))
    xs += list(rng.standard_normal(400) * np.exp2(rng.uniform(-12, 9, 400)))
    xs += [-m for m in mids[::7]] + [0.0, -0.0, 2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -11]
    got = O.e4m3_encode(np.array(xs))
    for x, c in zip(xs, got):
        assert int(c) == _brute_e4m3(x), (x, int(c))
    fin = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(fin)), fin)
    sat = O.e4m3_encode(np.array([448.0, 449.0, 463.9, 464.0, 1e6, np.inf, -500.0, -np.inf, np.nan]))
    assert list(sat) == [0x7E] * 6 + [0xFE, 0xFE, 0x7F]


@pytest.mark.parametrize("L,n,B,window", [(5, 2, 3, 0), (4, 3, 2, 3)])
def test_brute_force_tiny_fp8_cache(L, n, B, window):
    """The layer over an fp8 cache: appended rows stored as the exhaustively
    searched nearest E4M3 value of x / scale, times the scale, and attention
    over those stored values, against the scalar-loop formulation."""
    rng = np.random.default_rng(300 + L + n)
    p = _tiny_params(rng, window=window)
    d = p.w_qkv.shape[1]
    ks, vs = 0.375, 0.0625
    grid = np.concatenate([_e4m3_grid(), -_e4m3_grid()[1:]])
    K0 = rng.choice(grid, (p.n_kv, L, p.d_h)) * ks          # a cache already in fp8
    V0 = rng.choice(grid, (p.n_kv, L, p.d_h)) * vs
    C, H = rng.standard_normal((n, d)), rng.standard_normal((B, d))

    def q8(scale):
        def f(row):
            return [float(O.e4m3_decode(np.uint8(_brute_e4m3(t / scale)))) * scale for t in row]
        return f

    res = O.kv_inject_layer(p, K0, V0, C, H, kv_scales=(ks, vs))
    out, Kc, Vc = _brute_layer(p, K0, V0, C, H, q8(ks), q8(vs))
    assert np.max(np.abs(res.K - np.array(Kc))) == 0.0 and np.max(np.abs(res.V - np.array(Vc))) == 0.0
    assert np.max(np.abs(res.out - out)) < 1e-12
    exact = O.kv_inject_layer(p, K0, V0, C, H)
    assert np.max(np.abs(exact.out - res.out)) > 1e-6   # fp8 storage does change the output


def test_fp8_cache_error_is_bounded():
    """Storing the new rows in fp8 moves every element by at most half a step
    of its binade (relative 2^-4 for normal values), and the walkthrough
    layer's output by a few percent, not more."""
    wl = configs.WALKTHROUGH
    p = _params(wl)
    rng = np.random.default_rng(9)
    d = p.w_qkv.shape[1]
    K0, V0 = rng.standard_normal((p.n_kv, 40, p.d_h)), rng.standard_normal((p.n_kv, 40, p.d_h))
    K0, V0 = O.e4m3_quantize(K0, 1.0), O.e4m3_quantize(V0, 1.0)
    C, H = rng.standard_normal((3, d)), rng.standard_normal((4, d))
    res = O.kv_inject_layer(p, K0, V0, C, H, kv_scales=(1.0, 1.0))
    exact = O.kv_inject_layer(p, K0, V0, C, H)
    for got, want in ((res.K[:, 40:], exact.K[:, 40:]), (res.V[:, 40:], exact.V[:, 40:])):
        big = np.abs(want) >= 2.0 ** -6
        assert np.all(np.abs(got - want)[big] <= 2.0 ** -4 * np.abs(want)[big])
        assert np.all(np.abs(got - want)[~big] <= 2.0 ** -10)
    e = np.linalg.norm(res.out - exact.out) / np.linalg.norm(exact.out)
    assert 1e-4 < e < 0.05, e


# ---------------------------------------------------------------- bookkeeping

def test_acceptance_example_and_state_update():
    a, s = GOLDEN["acceptance"], GOLDEN["state_update"]
    acc = O.acceptance_length(a["block"][1:], a["posterior_head"])
    assert acc == a["acceptance_length"]
    assert O.next_start(s["start_before"], acc) == s["start_after"]
    assert O.new_context_rows(acc) == s["new_context_rows"] == len(s["new_context_positions"])
    # identical and fully-mismatched blocks
    assert O.acceptance_length([1, 2, 3], [1, 2, 3]) == 3
    assert O.acceptance_length([9, 2, 3], [1, 2, 3]) == 0


def test_accept_round_batch():
    """The batched acceptance on the walkthrough's block (tokens as ids), with
    the posterior's last prediction (from position 6, never checked) an
    arbitrary token; the identical, first-mismatch and later-match cases;
    B = 1 (nothing drafted)."""
    a = GOLDEN["acceptance"]
    vocab = {w: i for i, w in enumerate(sorted(set(a["block"] + a["posterior_head"] + [a["correction"], "<x>"])))}
    block = [vocab[w] for w in a["block"]]
    post = [vocab[w] for w in a["posterior_head"]] + [vocab["<x>"]]
    draft = [block[1:], [5, 6, 7], [9, 6, 7], [5, 9, 7]]
    posterior = [post, [5, 6, 7, 8], [5, 6, 7, 8], [5, 6, 7, 8]]
    acc, rows, anchor = O.accept_round(draft, posterior)
    assert list(acc) == [a["acceptance_length"], 3, 0, 1]
    assert list(rows) == [GOLDEN["state_update"]["new_context_rows"], 4, 1, 2]
    assert list(anchor) == [vocab[a["correction"]], 8, 5, 6]
    acc, rows, anchor = O.accept_round(np.zeros((2, 0), dtype=np.int64), [[3], [4]])
    assert list(acc) == [0, 0] and list(rows) == [1, 1] and list(anchor) == [3, 4]


def test_cache_growth_over_two_rounds():
    """Round 1 injects the 3 prompt positions; after the crop the draft cache
    holds positions 0-2; round 2 injects 3 accepted positions: 0-5."""
    rng = np.random.default_rng(16)
    p = _tiny_params(rng)
    d = p.w_qkv.shape[1]
    kd = 3 * d
    w_fc, g_h = rng.standard_normal((d, kd)) / math.sqrt(kd), np.ones(d)
    st = O.OracleStack([p], w_fc, g_h, 1e-6, [[np.zeros((p.n_kv, 0, p.d_h))]], [[np.zeros((p.n_kv, 0, p.d_h))]])
    s = GOLDEN["state_update"]
    B = 4
    st.round(rng.standard_normal((3, kd)), [0, 3], rng.standard_normal((B, d)), B)
    assert st.lengths() == [len(s["draft_cache_positions_round1"])]
    st.round(rng.standard_normal((s["new_context_rows"], kd)), [0, 3], rng.standard_normal((B, d)), B)
    assert st.lengths() == [len(s["draft_cache_positions_round2"])]


def test_stack_single_layer_matches_layer():
    """A one-layer stack round is exactly ctx_project followed by the layer."""
    rng = np.random.default_rng(17)
    p = _tiny_params(rng)
    d = p.w_qkv.shape[1]
    w_fc = rng.standard_normal((d, 2 * d))
    K0, V0 = rng.standard_normal((p.n_kv, 4, p.d_h)), rng.standard_normal((p.n_kv, 4, p.d_h))
    x, H = rng.standard_normal((2, 2 * d)), rng.standard_normal((3, d))
    st = O.OracleStack([p], w_fc, np.ones(d), 1e-6, [[K0]], [[V0]])
    outs, _ = st.round(x, [0, 2], H, 3)
    res = O.kv_inject_layer(p, K0, V0, O.ctx_project(x, w_fc, np.ones(d), 1e-6), H)
    assert np.array_equal(outs[0], res.out)



def _uniform_stack_layers(rng, n_layers, d=8, n_h=4, n_kv=2, d_h=4):
    """Layers whose W_K is zero: every key is zero after QK-norm and RoPE, so
    every score is 0 and each query's output is the plain mean of the V rows it
    sees (softmax of equal scores)."""
    layers = []
    for _ in range(n_layers):
        p = _tiny_params(rng, d, n_h, n_kv, d_h)
        w = p.w_qkv.copy()
        w[n_h * d_h:(n_h + n_kv) * d_h] = 0.0
        layers.append(O.LayerParams(w, p.w_o, p.gamma_q, p.gamma_k, n_h, n_kv, d_h, p.eps, p.theta, 0))
    return layers


def test_stack_chaining_closed_form():
    """Layer stacks ("DFlash KV Injection Walkthrough" Step 2: one context C for
    every draft layer; reading R14: H_{l+1} = H_l + out_l, each layer its own
    cache, every layer cropped to L + n after the round).  With uniform
    attention (zero keys), request r's block rows in layer l all get
    out = mean_j(v_j) expanded to the query heads times W_O^T, where the v_j are
    layer l's V rows of its cached context, of this round's C rows of request r
    and of its block input H_l.  Two layers, two requests with ragged context
    rows (one round with n = 0), two rounds: the closed form below tracks each
    layer's V rows with plain matrix algebra and must match the stack's outputs,
    lengths and cached V rows."""
    rng = np.random.default_rng(31)
    n_layers, R, B, d = 2, 2, 2, 8
    layers = _uniform_stack_layers(rng, n_layers, d)
    n_h, n_kv, d_h = layers[0].n_h, layers[0].n_kv, layers[0].d_h
    w_fc = rng.standard_normal((d, 3 * d)) / math.sqrt(3 * d)
    gamma_h = 1 + 0.1 * rng.standard_normal(d)
    L0 = [3, 1]
    K0 = [[np.zeros((n_kv, L0[r], d_h)) for r in range(R)] for _ in range(n_layers)]
    V0 = [[rng.standard_normal((n_kv, L0[r], d_h)) for r in range(R)] for _ in range(n_layers)]
    st = O.OracleStack(layers, w_fc, gamma_h, 1e-6, K0, V0)
    vrows = [[V0[l][r].copy() for r in range(R)] for l in range(n_layers)]

    def v_of(p, x):   # V rows of x under layer p: [n_kv, rows, d_h]
        wv = np.asarray(p.w_qkv)[(n_h + n_kv) * d_h:]
        return (x @ wv.T).reshape(x.shape[0], n_kv, d_h).transpose(1, 0, 2)

    for rnd, n in enumerate([[2, 0], [1, 3]]):
        cu = [0, n[0], n[0] + n[1]]
        x = rng.standard_normal((cu[-1], 3 * d))
        H = rng.standard_normal((R * B, d))
        outs, _ = st.round(x, cu, H, B)
        C = O.ctx_project(x, w_fc, gamma_h, 1e-6)
        h = H.copy()
        for l, p in enumerate(layers):
            want = np.empty_like(h)
            for r in range(R):
                ctx = v_of(p, C[cu[r]:cu[r + 1]])
                keys = np.concatenate([vrows[l][r], ctx, v_of(p, h[r * B:(r + 1) * B])], axis=1)
                mean = keys.mean(axis=1)                                   # [n_kv, d_h]
                o = np.concatenate([mean[hq // (n_h // n_kv)] for hq in range(n_h)])
                want[r * B:(r + 1) * B] = o @ np.asarray(p.w_o).T
                vrows[l][r] = np.concatenate([vrows[l][r], ctx], axis=1)
            assert np.allclose(outs[l], want, rtol=0, atol=1e-12), f"round {rnd} layer {l}"
            h = h + want
        for l in range(n_layers):
            assert st.lengths(l) == [vrows[l][r].shape[1] for r in range(R)]
            for r in range(R):
                assert np.allclose(st.V[l][r], vrows[l][r], rtol=0, atol=1e-12)

# ---------------------------------------------------------------- draft head (Step 5)

def _head_inputs(rng, B, d, vocab):
    h = rng.standard_normal((B, d))
    gamma = 1 + 0.1 * rng.standard_normal(d)
    w = rng.standard_normal((vocab, d)) / math.sqrt(d)
    return h, gamma, w


def test_draft_head_keeps_the_last_rows():
    """Step 5: the block's 4 output rows [4, 512] give 3 rows of logits, those
    of positions 4-6; row 0 (the known token at position 3) does not enter.
    Negating block row j negates logits row j - 1 and nothing else (the norm
    and the product are odd in each row)."""
    wl = configs.WALKTHROUGH
    gh = GOLDEN["draft_head"]
    rng = np.random.default_rng(0)
    vocab = 50
    h, gamma, w = _head_inputs(rng, wl.B, wl.d, vocab)
    logits, ids = O.draft_head(h, gamma, wl.eps, w, wl.B)
    assert logits.shape == (gh["rows_kept"], vocab) and ids.shape == (gh["rows_kept"],)
    block_pos = GOLDEN["positions"]["q"]
    assert block_pos[1:] == gh["positions"]
    h0 = h.copy()
    h0[0] = 7.0 * rng.standard_normal(wl.d)
    assert np.array_equal(O.draft_head(h0, gamma, wl.eps, w, wl.B)[0], logits)
    for j in range(1, wl.B):
        hj = h.copy()
        hj[j] = -hj[j]
        lj, _ = O.draft_head(hj, gamma, wl.eps, w, wl.B)
        for i in range(wl.B - 1):
            assert np.allclose(lj[i], -logits[i] if i == j - 1 else logits[i], rtol=0, atol=1e-12)


def test_draft_head_closed_forms():
    """lm_head rows that are permuted unit vectors read single normed entries:
    with every |h| entry equal to a, RMSNorm divides by a, so logit j of a row
    is sign(h[pi(j)]) * gamma[pi(j)] (pi the permutation); requests are
    independent blocks of B rows; the argmax is the first maximal logit."""
    rng = np.random.default_rng(1)
    d, B, R = 16, 3, 2
    a = 2.5
    signs = rng.choice([-1.0, 1.0], size=(R * B, d))
    h = a * signs
    gamma = 1.0 + np.arange(d) / 8.0
    pi = rng.permutation(d)
    w = np.eye(d)[pi]                       # row j = e_{pi(j)}
    logits, ids = O.draft_head(h, gamma, 0.0, w, B)
    rows = [r * B + 1 + j for r in range(R) for j in range(B - 1)]
    want = signs[rows][:, pi] * gamma[pi][None, :]
    assert np.allclose(logits, want, rtol=1e-15, atol=0)
    assert list(ids) == [int(np.argmax(want[i])) for i in range(len(rows))]
    # ties: two lm_head rows equal to the row holding the maximum -> the lower index
    top = int(ids[0])
    w2 = np.vstack([w, w[top:top + 1]])
    _, ids2 = O.draft_head(h, gamma, 0.0, w2, B)
    assert ids2[0] == top and top < d
