"""Device-driven rounds ("DFlash KV Injection Walkthrough" Steps 6 and 7): the
acceptance of each round (dflash_accept, on the device) decides how many
context rows the next round injects, and the cache is cut back on the device,
so a whole sequence of rounds runs with no host read and is captured in one HIP
graph.  The draft and target tokens of each round are seeded with a planted
match prefix of k positions, so the host knows every round's acceptance
(k + 1 new rows next round) in advance and the fp64 oracle can run the same
rounds.  Checked: every round's output against the oracle (the bf16 bar), the
lengths after the rounds bit for bit against the rows appended, the block
tables against the integer cache model fed with the bound sequence the host
plans for, and the cached context rows against the oracle's."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU visible", allow_module_level=True)

from block_diffusion_draft_fc_amd import _lib as L  # noqa: E402
from oracle import cache_model as CM  # noqa: E402
from workloads import configs, generate as G  # noqa: E402
from workloads.device import from_device, to_device  # noqa: E402

from gpu_harness import TOL, cache_rows, oracle_stack, prefill_host, rel_l2, say  # noqa: E402

VOCAB = 32000


def _device_rounds(wl, rounds, n0):
    """Runs `rounds` device-driven rounds of a one-layer workload captured in
    one graph; returns (per-round GPU outputs, per-round n, cache, model)."""
    R, B, n_max = wl.R, wl.B, wl.B
    kv = prefill_host(wl)
    L0 = [int(x) for x in G.prefill_lengths(wl)]
    # the rounds' new rows: round 0 from the argument, round i+1 the planted
    # acceptance of round i plus one
    toks = [G.accept_tokens(wl.seed, R, B, VOCAB, rnd=i) for i in range(rounds)]
    ns = [list(n0)] + [[int(t[2][r]) + 1 for r in range(R)] for t in toks[:-1]]
    fc, lw = G.fc_weights(wl), G.layer_weights(wl, 0)
    w_fc, g_h = to_device(fc["w_fc"], wl), to_device(fc["gamma_h"], wl)
    layer = L.Layer(*(to_device(lw[k], wl) for k in ("w_qkv", "w_o", "gamma_q", "gamma_k")),
                    n_h=wl.n_h, n_kv=wl.n_kv, d_h=wl.d_h, eps=wl.eps, rope_theta=wl.rope_theta)
    bound = [L0[r] + rounds * n_max + B for r in range(R)]
    if wl.page_size:
        ps = wl.page_size
        pages = sum(-(-b // ps) for b in bound) + R
        maxp = max(-(-b // ps) for b in bound) + 1
        cache = L.Cache(R, wl.n_kv, wl.d_h, torch.bfloat16, pages, ps, maxp, "cuda")
        model = CM.CacheModel(R, wl.n_kv, wl.d_h, ps, pages, maxp)
    else:
        cap = (max(bound) + 63) // 64 * 64
        cache = L.Cache(R, wl.n_kv, wl.d_h, torch.bfloat16, cap, device="cuda")
        model = CM.CacheModel(R, wl.n_kv, wl.d_h, 0, cap)
    cu = [0]
    for r in range(R):
        cu.append(cu[-1] + L0[r])
    kr = np.concatenate([kv[0][r][0].transpose(1, 0, 2) for r in range(R)], axis=0)
    vr = np.concatenate([kv[0][r][1].transpose(1, 0, 2) for r in range(R)], axis=0)
    L.dflash_cache_append(cache, cu, to_device(kr, wl), to_device(vr, wl))
    zeros = np.zeros((cu[-1], wl.n_kv, wl.d_h), dtype=np.uint16)
    model.append(cu, zeros, zeros)

    xs, Hs, outs, drafts, posts = [], [], [], [], []
    for i in range(rounds):
        x, xcu, H = G.round_inputs(wl, i, ns[i])
        pad = np.zeros((R * n_max, wl.kd), dtype=np.float32)
        for r in range(R):
            pad[r * n_max:r * n_max + ns[i][r]] = x[xcu[r]:xcu[r + 1]]
        xs.append(to_device(pad, wl))
        Hs.append(to_device(H, wl))
        outs.append(torch.full((R * B, wl.d), float("nan"), dtype=torch.bfloat16, device="cuda"))
        drafts.append(torch.from_numpy(toks[i][0].reshape(-1).copy()).cuda())
        posts.append(torch.from_numpy(toks[i][1]).cuda())
    Cb = torch.empty((R * n_max, wl.d), dtype=torch.bfloat16, device="cuda")
    cws = torch.empty(L.dflash_ctx_project_ws_bytes(R * n_max, wl.kd, wl.d, torch.bfloat16), dtype=torch.uint8,
                      device="cuda")
    ws = torch.empty(L.dflash_kv_inject_attn_dev_ws_bytes(layer, cache, n_max, B), dtype=torch.uint8, device="cuda")
    d_len = torch.full((R,), -1, dtype=torch.int32, device="cuda")
    d_rows = torch.tensor(ns[0], dtype=torch.int32, device="cuda")
    acc = torch.empty((R,), dtype=torch.int32, device="cuda")
    L.dflash_cache_device_begin(cache, d_len)
    torch.cuda.synchronize()
    say(f"case {wl.name}: capturing {rounds} device-driven rounds in one graph")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(rounds):
            L.dflash_ctx_project(xs[i], w_fc, g_h, wl.eps, Cb, cws)
            L.dflash_kv_inject_attn_dev(layer, cache, Cb, n_max, d_rows, Hs[i], B, outs[i], ws)
            L.dflash_cache_crop_tail_dev(cache, B)
            L.dflash_accept(drafts[i], posts[i], acc, d_rows)
    # the host planned for the bounds: every round n_max new rows
    for i in range(rounds):
        z = np.zeros((R * (n_max + B), wl.n_kv, wl.d_h), dtype=np.uint16)
        model.append([r * (n_max + B) for r in range(R + 1)], z, z)
        model.crop([model.len[r] - B for r in range(R)])
    assert cache.lengths() == model.len
    g.replay()
    torch.cuda.synchronize()
    L.dflash_cache_device_end(cache)
    true_len = [L0[r] + sum(ns[i][r] for i in range(rounds)) for r in range(R)]
    model.crop(true_len)
    assert cache.lengths() == true_len, f"{cache.lengths()} != {true_len}"
    assert d_rows.cpu().tolist() == [int(toks[-1][2][r]) + 1 for r in range(R)]
    if wl.page_size:
        assert cache.block_table() == [p + [-1] * (cache.max_pages - len(p)) for p in model.block_table()]
        assert L.LIB.dflash_cache_free_pages(cache.handle) == len(model.free)
    return [from_device(o) for o in outs], ns, cache, kv


def _check_against_oracle(wl, rounds, n0):
    got, ns, cache, kv = _device_rounds(wl, rounds, n0)
    orc = oracle_stack(wl, kv)
    worst = 0.0
    for i in range(rounds):
        x, cu, H = G.round_inputs(wl, i, ns[i])
        ref, _ = orc.round(x, cu, H, wl.B)
        e = rel_l2(got[i], ref[0])
        worst = max(worst, e)
        assert e <= TOL["bf16"], f"round {i}: rel-L2 {e:.3e}"
    assert orc.lengths(0) == cache.lengths()
    L0 = G.prefill_lengths(wl)
    for r in range(wl.R):
        K, V = cache_rows(cache, r)
        a = int(L0[r])
        assert rel_l2(K[:, a:], orc.K[0][r][:, a:]) <= TOL["bf16"]
        assert rel_l2(V[:, a:], orc.V[0][r][:, a:]) <= TOL["bf16"]
    say(f"  {rounds} rounds, worst rel-L2 {worst:.3e}, lengths {cache.lengths()}")


def test_device_driven_decode_8k_64_rounds_one_graph():
    """The 8K decode workload's layer: 64 rounds in one HIP graph, each round's
    new rows decided by the previous round's acceptance on the device."""
    wl = configs.DECODE_8K
    _check_against_oracle(wl, 64, [int(G.schedule(wl)[0][0])])


def test_device_driven_paged_ragged_one_graph():
    """Four requests of ragged lengths on a paged cache of 64-row pages, pages
    reserved for the bounds: 12 rounds in one graph, block tables against the
    integer model."""
    wl = configs.WALKTHROUGH.scaled(name="device_rounds_paged_ragged", d=256, n_h=8, n_kv=2, d_h=64, k_layers=2,
                                    B=4, R=4, rounds=12, dtype="bf16", seed=13, prefill="uniform",
                                    prefill_range=(40, 300), n_new="uniform", n_range=(1, 4),
                                    block_rows="anchor_mask", page_size=64)
    _check_against_oracle(wl, 12, [1, 4, 2, 3])


def test_device_mode_refuses_host_calls():
    wl = configs.WALKTHROUGH.scaled(name="device_mode_refusals", d=256, n_h=8, n_kv=2, d_h=64, dtype="bf16")
    cache = L.Cache(1, wl.n_kv, wl.d_h, torch.bfloat16, 128, device="cuda")
    d_len = torch.zeros((1,), dtype=torch.int32, device="cuda")
    L.dflash_cache_device_begin(cache, d_len)
    k = torch.zeros((4, wl.n_kv, wl.d_h), dtype=torch.bfloat16, device="cuda")
    assert L.LIB.dflash_cache_append(cache.handle, L._i32([0, 4]), k.data_ptr(), k.data_ptr(), None) == L.ERR_ARG
    assert L.LIB.dflash_cache_crop(cache.handle, L._i32([0]), None) == L.ERR_ARG
    assert L.LIB.dflash_cache_device_begin(cache.handle, d_len.data_ptr(), None) == L.ERR_ARG
    L.dflash_cache_device_end(cache)
    assert cache.lengths() == [0]
    assert L.LIB.dflash_cache_crop_tail_dev(cache.handle, 4, None) == L.ERR_ARG
    assert L.LIB.dflash_cache_device_end(cache.handle, None) == L.ERR_ARG


def test_device_rows_out_of_range_act_as_the_bounds():
    """Row counts on the device are clamped to 0..n_max by every kernel that
    reads them: a round given [n_max + 7, -3] matches the round given
    [n_max, 0] (outputs bit for bit, lengths), so a bad count cannot move a
    read or write past the planned bounds."""
    wl = configs.WALKTHROUGH.scaled(name="device_rows_clamped", d=256, n_h=8, n_kv=2, d_h=64, k_layers=2, B=4,
                                    R=2, rounds=1, dtype="bf16", seed=17, prefill="fixed", prefill_len=100,
                                    n_new="fixed", n_fixed=4, block_rows="anchor_mask")
    R, B, n_max = wl.R, wl.B, 4
    kv = prefill_host(wl)
    fc, lw = G.fc_weights(wl), G.layer_weights(wl, 0)
    w_fc, g_h = to_device(fc["w_fc"], wl), to_device(fc["gamma_h"], wl)
    layer = L.Layer(*(to_device(lw[k], wl) for k in ("w_qkv", "w_o", "gamma_q", "gamma_k")),
                    n_h=wl.n_h, n_kv=wl.n_kv, d_h=wl.d_h, eps=wl.eps, rope_theta=wl.rope_theta)
    x, _, H = G.round_inputs(wl, 0, [n_max] * R)
    xd, Hd = to_device(x, wl), to_device(H, wl)
    kr = np.concatenate([kv[0][r][0].transpose(1, 0, 2) for r in range(R)], axis=0)
    vr = np.concatenate([kv[0][r][1].transpose(1, 0, 2) for r in range(R)], axis=0)
    results = []
    for rows in ([n_max + 7, -3], [n_max, 0]):
        say(f"case {wl.name}: d_rows {rows}")
        cache = L.Cache(R, wl.n_kv, wl.d_h, torch.bfloat16, 256, device="cuda")
        L.dflash_cache_append(cache, [0, 100, 200], to_device(kr, wl), to_device(vr, wl))
        C = torch.empty((R * n_max, wl.d), dtype=torch.bfloat16, device="cuda")
        cws = torch.empty(L.dflash_ctx_project_ws_bytes(R * n_max, wl.kd, wl.d, torch.bfloat16),
                          dtype=torch.uint8, device="cuda")
        ws = torch.empty(L.dflash_kv_inject_attn_dev_ws_bytes(layer, cache, n_max, B), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty((R * B, wl.d), dtype=torch.bfloat16, device="cuda")
        d_len = torch.zeros((R,), dtype=torch.int32, device="cuda")
        d_rows = torch.tensor(rows, dtype=torch.int32, device="cuda")
        L.dflash_cache_device_begin(cache, d_len)
        L.dflash_ctx_project(xd, w_fc, g_h, wl.eps, C, cws)
        L.dflash_kv_inject_attn_dev(layer, cache, C, n_max, d_rows, Hd, B, out, ws)
        torch.cuda.synchronize()
        lengths = d_len.cpu().tolist()
        L.dflash_cache_device_end(cache)
        K, V = cache_rows(cache, 0)
        results.append((out.cpu(), lengths, K, V))
    assert results[0][1] == results[1][1] == [100 + n_max + B, 100 + B]
    assert torch.equal(results[0][0], results[1][0])
    assert np.array_equal(results[0][2], results[1][2]) and np.array_equal(results[0][3], results[1][3])
