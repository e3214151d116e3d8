"""Plant plausible mistakes in the oracle (on the CPU, by monkeypatching) and
check that the pins catch every one: a dropped term, a wrong sign or index, a
transposed operand, a wrong scale, a causal mask, a wrong RoPE offset."""
import numpy as np
import pytest

from oracle import dflash_oracle as O
import tests.test_oracle as T

PINS = [
    T.test_walkthrough_shapes_and_positions,
    T.test_scaling_is_printed_value,
    T.test_softmax_rows_sum_to_one_and_no_causal_mask,
    T.test_rmsnorm_closed_forms,
    T.test_ctx_project_brute_force,
    T.test_rope_equals_complex_rotation,
    T.test_rope_group_properties,
    lambda: T.test_rope_relative_position_invariance(8192),
    T.test_rope_example_pair_and_wrong_offset,
    T.test_layer_tail_offset_matters,
    T.test_gqa_equals_repeated_kv_mha,
    T.test_position_zero_reduces_to_library_sdpa,
    T.test_single_key_closed_form,
    T.test_dual_stream_rows_are_independent,
    T.test_window_closed_forms,
    lambda: T.test_brute_force_tiny(5, 1, 3, 0),
    lambda: T.test_brute_force_tiny(4, 3, 3, 3),
    lambda: T.test_brute_force_tiny(5, 2, 1, 1),
    T.test_cache_growth_over_two_rounds,
    T.test_draft_head_keeps_the_last_rows,
    T.test_draft_head_closed_forms,
    T.test_acceptance_example_and_state_update,
    T.test_accept_round_batch,
    T.test_e4m3_format_values,
    T.test_e4m3_matches_library_cast,
    T.test_e4m3_encode_brute_force_and_ties,
    lambda: T.test_brute_force_tiny_fp8_cache(5, 2, 3, 0),
    T.test_fp8_cache_error_is_bounded,
    T.test_stack_single_layer_matches_layer,
    T.test_stack_chaining_closed_form,
]

_encode, _decode = O.e4m3_encode, O.e4m3_decode


def _enc_rounding(rnd, saturate=True):
    def enc(x):
        x = O.f64(x)
        a = np.abs(x)
        if saturate:
            a = np.minimum(a, 448.0)
        _, k = np.frexp(a)
        e = np.where(a < 2.0 ** -6, -6, k - 1)
        q = rnd(np.where(np.isnan(a), 0.0, a) * np.exp2(3.0 - e))
        bits = np.minimum((e + 6) * 8 + q.astype(np.int64), 0x7F)
        bits = np.where(np.signbit(x), bits | 0x80, bits)
        return np.where(np.isnan(x), 0x7F, bits).astype(np.uint8)
    return enc


def _dec_bias8(codes):
    return _decode(codes) / 2.0


def _dec_subnormal_hidden_one(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    v = _decode(codes)
    sub = ((c >> 3) & 15) == 0
    return np.where(sub, np.where(c & 0x80, -1.0, 1.0) * (1.0 + (c & 7) / 8.0) * 2.0 ** -6, v)


def _quant_nothing(x, scale):
    return O.f64(x)


def _quant_scale_multiplied(x, scale):
    return _decode(_encode(O.f64(x) * scale)) / scale


def _rope_sign(x, positions, theta):
    x = O.f64(x); half = x.shape[-1] // 2
    ang = O.f64(positions)[:, None] * O.rope_inv_freq(x.shape[-1], theta)[None, :]
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * np.cos(ang) + hi * np.sin(ang), hi * np.cos(ang) - lo * np.sin(ang)], -1)


def _rope_interleaved(x, positions, theta):
    x = O.f64(x)
    ang = O.f64(positions)[:, None] * O.rope_inv_freq(x.shape[-1], theta)[None, :]
    ev, od = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = ev * np.cos(ang) - od * np.sin(ang)
    y[..., 1::2] = od * np.cos(ang) + ev * np.sin(ang)
    return y


def _attn_factory(head_map=None, scale_pow=-0.5, causal=False):
    def attn(q, K, V, qpos, kpos, window=0):
        q, K, V = O.f64(q), O.f64(K), O.f64(V)
        n_h, B, d_h = q.shape
        n_kv, L_tot, _ = K.shape
        vis = O.visible(qpos, kpos, window)
        if causal:
            vis = vis & (np.asarray(kpos)[None, :] <= np.asarray(qpos)[:, None])
        o = np.empty((n_h, B, d_h)); A = np.empty((n_h, B, L_tot))
        for h in range(n_h):
            g = head_map(h, n_h, n_kv) if head_map else h // (n_h // n_kv)
            s = np.where(vis, (q[h] @ K[g].T) * d_h ** scale_pow, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            A[h] = e / e.sum(axis=1, keepdims=True)
            o[h] = A[h] @ V[g]
        return o, A
    return attn


def _kv_no_knorm(p, C, H):
    _, wk, wv = p.split()
    S = np.concatenate([O.f64(C), O.f64(H)], axis=0)
    k = (S @ wk.T).reshape(S.shape[0], p.n_kv, p.d_h)
    v = (S @ wv.T).reshape(S.shape[0], p.n_kv, p.d_h)
    return k.transpose(1, 0, 2), v.transpose(1, 0, 2)


def _kv_block_first(p, C, H):
    return _ORIG["project_kv"](p, H, C)


def _rms_no_gamma(x, gamma, eps):
    x = O.f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _rms_no_eps(x, gamma, eps):
    x = O.f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) * O.f64(gamma)


def _rms_sum(x, gamma, eps):
    x = O.f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * O.f64(gamma)


def _ctx_transposed(x_raw, w_fc, gamma_h, eps):
    w = O.f64(w_fc)
    return O.rms_norm(O.f64(x_raw) @ w.reshape(w.shape[1], w.shape[0]), gamma_h, eps)


def _oproj_head_minor(o, w_o):
    o = O.f64(o); n_h, B, d_h = o.shape
    return o.transpose(1, 2, 0).reshape(B, n_h * d_h) @ O.f64(w_o).T


def _crop_keep_block(K, V, new_len):
    return K, V


def _window_inclusive(qpos, kpos, window):
    qpos, kpos = np.asarray(qpos), np.asarray(kpos)
    if window <= 0:
        return np.ones((qpos.size, kpos.size), dtype=bool)
    return (qpos[:, None] - kpos[None, :]) <= window


def _inv_freq_wrong(d_h, theta):
    i = np.arange(d_h // 2, dtype=np.float64)
    return np.power(float(theta), -i / d_h)


def _layer_q_front(p, K_cache, V_cache, C, H, kv_scales=None):
    res = _ORIG["kv_inject_layer"](p, K_cache, V_cache, C, H, kv_scales)
    L = np.asarray(K_cache).shape[1]
    qpos = L + np.arange(H.shape[0])
    q = O.rope(O.project_q(p, H), qpos, p.theta)
    o, A = O.gqa_attention(q, res.K, res.V, qpos, res.kpos, p.window)
    return O.LayerResult(O.o_proj(o, p.w_o), res.K, res.V, q, A, qpos, res.kpos)


def _head_first_rows(h, gamma_f, eps, w_lm, B):
    h = O.f64(h); R = h.shape[0] // B
    x = O.rms_norm(h, gamma_f, eps).reshape(R, B, -1)[:, :-1, :].reshape(R * (B - 1), -1)
    logits = x @ O.f64(w_lm).T
    return logits, np.argmax(logits, axis=-1)


def _head_no_norm(h, gamma_f, eps, w_lm, B):
    h = O.f64(h); R = h.shape[0] // B
    x = (h * O.f64(gamma_f)).reshape(R, B, -1)[:, 1:, :].reshape(R * (B - 1), -1)
    logits = x @ O.f64(w_lm).T
    return logits, np.argmax(logits, axis=-1)


def _head_weight_columns(h, gamma_f, eps, w_lm, B):
    h = O.f64(h); R = h.shape[0] // B
    x = O.rms_norm(h, gamma_f, eps).reshape(R, B, -1)[:, 1:, :].reshape(R * (B - 1), -1)
    w = O.f64(w_lm)
    logits = x @ w.reshape(w.shape[1], w.shape[0])
    return logits, np.argmax(logits, axis=-1)


def _head_last_max(h, gamma_f, eps, w_lm, B):
    logits, _ = _ORIG["draft_head"](h, gamma_f, eps, w_lm, B)
    return logits, logits.shape[1] - 1 - np.argmax(logits[:, ::-1], axis=-1)


def _accept_counts_every_match(draft_tail, posterior_head):
    return int(sum(a == b for a, b in zip(draft_tail, posterior_head)))


def _accept_round_shifted(draft_ids, posterior):
    # the draft compared with the posterior of its own position, not the one before
    posterior = np.asarray(posterior)
    draft_ids = np.asarray(draft_ids).reshape(len(posterior), -1)
    acc = np.array([O.acceptance_length(list(draft_ids[r]), list(posterior[r][1:])) for r in range(len(posterior))])
    return acc, acc + 1, np.array([posterior[r][acc[r]] for r in range(len(posterior))])


def _accept_round_anchor_after(draft_ids, posterior):
    acc, rows, _ = _ORIG["accept_round"](draft_ids, posterior)
    posterior = np.asarray(posterior)
    return acc, rows, np.array([posterior[r][min(acc[r] + 1, posterior.shape[1] - 1)] for r in range(len(acc))])


def _stack_round_factory(no_residual=False, shared_cache=False, crop_last_only=False, ctx_first_layer_only=False):
    # OracleStack.round with one chaining mistake (caches of bf16/f32 values only)
    def round_(self, x_raw, cu, H, B):
        R = len(cu) - 1
        C = O.ctx_project(x_raw, self.w_fc, self.gamma_h, self.eps)
        h = O.f64(H).copy()
        outs, last = [], []
        for li, p in enumerate(self.layers):
            ci = 0 if shared_cache else li
            out_l = np.empty_like(h)
            res_l = []
            for r in range(R):
                L = self.K[ci][r].shape[1]
                ctx = C[cu[r]:cu[r + 1]] if (li == 0 or not ctx_first_layer_only) else C[:0]
                res = O.kv_inject_layer(p, self.K[ci][r], self.V[ci][r], ctx, h[r * B:(r + 1) * B])
                out_l[r * B:(r + 1) * B] = res.out
                n = cu[r + 1] - cu[r]
                if crop_last_only and li != len(self.layers) - 1:
                    self.K[ci][r], self.V[ci][r] = res.K, res.V
                else:
                    self.K[ci][r], self.V[ci][r] = O.crop(res.K, res.V, L + n)
                res_l.append(res)
            outs.append(out_l)
            last = res_l
            h = out_l if no_residual else h + out_l
        return outs, last
    return round_


_ORIG = {name: getattr(O, name) for name in
         ("rope", "gqa_attention", "project_kv", "rms_norm", "ctx_project", "o_proj",
          "crop", "visible", "rope_inv_freq", "kv_inject_layer", "draft_head", "accept_round")}

MUTANTS = {
    "rope_sign_flipped": ("rope", _rope_sign),
    "rope_interleaved_pairs": ("rope", _rope_interleaved),
    "rope_freq_exponent": ("rope_inv_freq", _inv_freq_wrong),
    "gqa_head_modulo": ("gqa_attention", _attn_factory(head_map=lambda h, n_h, n_kv: h % n_kv)),
    "scale_one_over_d": ("gqa_attention", _attn_factory(scale_pow=-1.0)),
    "causal_mask": ("gqa_attention", _attn_factory(causal=True)),
    "no_k_norm": ("project_kv", _kv_no_knorm),
    "block_rows_first": ("project_kv", _kv_block_first),
    "rmsnorm_no_gamma": ("rms_norm", _rms_no_gamma),
    "rmsnorm_no_eps": ("rms_norm", _rms_no_eps),
    "rmsnorm_sum_not_mean": ("rms_norm", _rms_sum),
    "fc_weight_transposed": ("ctx_project", _ctx_transposed),
    "oproj_head_minor": ("o_proj", _oproj_head_minor),
    "crop_does_nothing": ("crop", _crop_keep_block),
    "window_inclusive": ("visible", _window_inclusive),
    "queries_on_window_front": ("kv_inject_layer", _layer_q_front),
    "head_first_rows": ("draft_head", _head_first_rows),
    "head_no_norm": ("draft_head", _head_no_norm),
    "head_weight_columns": ("draft_head", _head_weight_columns),
    "head_last_maximum": ("draft_head", _head_last_max),
    "accept_counts_every_match": ("acceptance_length", _accept_counts_every_match),
    "accept_posterior_shifted": ("accept_round", _accept_round_shifted),
    "accept_anchor_one_late": ("accept_round", _accept_round_anchor_after),
    "e4m3_ties_away": ("e4m3_encode", _enc_rounding(lambda q: np.floor(q + 0.5))),
    "e4m3_truncates": ("e4m3_encode", _enc_rounding(np.floor)),
    "e4m3_no_saturation": ("e4m3_encode", _enc_rounding(np.rint, saturate=False)),
    "e4m3_bias_8": ("e4m3_decode", _dec_bias8),
    "e4m3_subnormal_hidden_one": ("e4m3_decode", _dec_subnormal_hidden_one),
    "fp8_cache_not_quantized": ("e4m3_quantize", _quant_nothing),
    "fp8_scale_inverted": ("e4m3_quantize", _quant_scale_multiplied),
    "stack_no_residual": ("OracleStack.round", _stack_round_factory(no_residual=True)),
    "stack_layers_share_one_cache": ("OracleStack.round", _stack_round_factory(shared_cache=True)),
    "stack_only_last_layer_cropped": ("OracleStack.round", _stack_round_factory(crop_last_only=True)),
    "stack_context_into_first_layer_only": ("OracleStack.round", _stack_round_factory(ctx_first_layer_only=True)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    owner = O
    if "." in attr:
        cls, attr = attr.split(".")
        owner = getattr(O, cls)
    monkeypatch.setattr(owner, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(getattr(pin, "__name__", "pin"))
    assert caught, f"mutant {name} survived every pin"
