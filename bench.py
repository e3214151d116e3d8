#!/usr/bin/env python3
"""Draft-round throughput of the DFlash KV-injection attention layer on one MI355X.

Workload: one Qwen3-8B-shaped draft attention layer in steady-state decode
(d 4096, 32 query / 8 K/V heads of 128, k = 5 target layers -> 20480-wide raw
context, block of 16, bf16 storage with fp32 accumulation, batch 1).  The draft
KV cache starts at 8192 rows; each round appends 1..16 newly accepted context
rows (seeded schedule of 64 rounds) plus the block, attends, and is cropped back
to the accepted prefix.  Step i runs round i mod 64; every 64 steps the cache is
cropped back to 8192 rows, so every step sees an 8.2K-8.7K-key cache.

One step = dflash_ctx_project (fc + hidden_norm) + dflash_kv_inject_attn
(q/k/v projections, QK-norm, RoPE, cache append, attention, o_proj) +
dflash_cache_crop.  All inputs are resident in HBM before timing starts.

Prints one JSON line: draft blocks/s (value), the attention kernel's HBM
throughput against the 8 TB/s peak (roofline), per-stage times from HIP events
recorded on the launch stream, and the fp64 CPU oracle timed on a bounded
sample of the same rounds (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
METRIC = "draft blocks/sec + attn HBM GB/s (% peak), ctx 8K, block 16, GQA 32/8"


def head_start(calls: int, us_per_call: float = 100.0) -> None:
    """Enqueue register-only MFMA work (no memory traffic) before an
    event-timed eager loop of `calls` library calls: while it runs, the host
    enqueues the loop ahead of the GPU.  A kernel-attached event pair stamps
    its start when the stream reaches the launch, so a host that falls behind
    the GPU adds its submission gap to the kernel's time; with the head start
    the loop's kernels run back to back and the events bracket the kernels
    alone (the rocprofv3 kernel trace measures the same launches the same).
    About us_per_call of head start per call, at most 40 ms; ~13000
    iterations of the 256-workgroup MFMA loop take a millisecond."""
    from block_diffusion_draft_fc_amd import _lib as L

    ms = min(40.0, calls * us_per_call * 1e-3)
    if ms > 0:
        L.dflash_mfma_peak(max(1, int(ms * 13000)), 256)


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--mode", choices=("best", "graph", "eager"), default="best",
                    help="graph: the rounds' launches replayed from captured HIP graphs (one per 64-round "
                         "cycle); eager: issued by the library calls; best: time both, report the faster")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fresh-ctx", action="store_true",
                    help="skip the MFMA-utilisation pass over the fresh 1024-row context projections")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip the attention-at-scale pass, the draft head, the acceptance, the ragged 16-request "
                         "and the 5-layer hybrid stack rounds")
    ap.add_argument("--attn-pass", metavar="R,CTX,KV",
                    help="only time the attention kernel for R requests of CTX cached keys with a KV "
                         "(bf16 or fp8) cache, print its JSON and exit (for profiling one kernel)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 8 times (scales HBM counters)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="no GPU work: read the rocprofv3 outputs under DIR (prof_decode/, pmc_FETCH_SIZE/, "
                         "pmc_WRITE_SIZE/, pmc_copy_FETCH_SIZE/, pmc_copy_WRITE_SIZE/ as written by the commands "
                         "in profiles/) and write the kernel-trace and HBM-traffic summaries into profiles/")
    return ap.parse_args()


def copy_calibration():
    """A plain copy kernel of known size: 256 MiB read and 256 MiB written per
    launch, so per-dispatch FETCH_SIZE / WRITE_SIZE should read 262144 KiB."""
    import torch

    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(8):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 8}), flush=True)
    return 0


# ---------------------------------------------------------------------------- algorithmic work

def round_work(wl, L, n):
    """Algorithmic bytes / FLOPs of one round at cache length L with n new rows:
    every tensor the method must touch, moved once."""
    eb = 2
    B, d, kd = wl.B, wl.d, wl.kd
    qd, kvd = wl.n_h * wl.d_h, wl.n_kv * wl.d_h
    L_tot = L + n + B
    w = {}
    w["ctx_gemm"] = dict(bytes=(d * kd + n * kd + n * d) * eb, flops=2 * n * kd * d)
    w["qkv_gemm"] = dict(bytes=((qd + 2 * kvd) * d + (n + B) * d) * eb, flops=2 * (B * qd + (n + B) * 2 * kvd) * d)
    # attention: every cached K and V row once, the queries once
    w["attn"] = dict(bytes=(L_tot * 2 * kvd + B * qd) * eb, flops=4 * wl.n_h * B * L_tot * wl.d_h)
    w["o_gemm"] = dict(bytes=(d * qd + B * qd + B * d) * eb, flops=2 * B * qd * d)
    w["round"] = dict(bytes=sum(v["bytes"] for v in w.values()), flops=sum(v["flops"] for v in w.values()))
    return w


# ---------------------------------------------------------------------------- HBM traffic record

ATTN_SOURCES = ("attention.hip", "attn_merge.hpp")


def attention_source_sha256():
    """SHA-256 over the bf16 attention kernel's sources (the kernel file and
    the merge helpers it includes), in that order."""
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        h.update(open(os.path.join(ROOT, "block_diffusion_draft_fc_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def traffic_record():
    """Measured HBM bytes per attention launch (rocprofv3 FETCH_SIZE + WRITE_SIZE,
    scaled by a plain copy's reading), from the record kept with the profiles -
    or None when the attention kernel's source has changed since it was taken."""
    rec_path = os.path.join(ROOT, "profiles", "attn_decode_ctx8k_traffic.json")
    try:
        rec = json.load(open(rec_path))
        sha = attention_source_sha256()
    except (OSError, ValueError):
        return None
    if rec.get("attention_source_sha256") != sha:
        return None
    return int(rec["fetch_bytes_per_launch"]) + int(rec["write_bytes_per_launch"])


# ---------------------------------------------------------------------------- CPU oracle leg

def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


PARITY_ROUNDS = 8   # rounds of the cycle the CPU leg also checks against the GPU's outputs


def cpu_baseline(wl, budget_s, gpu_outs=()):
    """The fp64 oracle on the host cores, over the first rounds of the same
    schedule until `budget_s` seconds of round work have run with every
    BLAS thread, then a third of that budget on one thread.  The oracle's
    prefill (building its cache of the 8192 prefilled rows) is timed apart.
    gpu_outs[r]: the layer output of round r from the GPU (rounds in order
    from the same prefill); their rel-L2 against the oracle's outputs of the
    same rounds is reported as `parity` (outside the timed round work)."""
    from oracle import dflash_oracle as O
    from workloads import generate as G

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits, blas = None, 1
    cores = len(os.sched_getaffinity(0))
    fc, lw = G.fc_weights(wl), G.layer_weights(wl, 0)
    p = O.LayerParams(lw["w_qkv"].astype(np.float64), lw["w_o"].astype(np.float64), lw["gamma_q"],
                      lw["gamma_k"], wl.n_h, wl.n_kv, wl.d_h, wl.eps, wl.rope_theta, 0)
    K0, V0 = G.prefill_kv(wl, 0, 0, wl.prefill_len)
    sched = G.schedule(wl)

    errs = []

    def run(budget, check=False):
        """Rounds of the cycle in order (starting over from the prefill after
        round 63) until `budget` seconds of round work."""
        done, spent, prefill_s = 0, 0.0, 0.0
        while spent < budget:
            r = done % wl.rounds
            if r == 0:
                t0 = time.perf_counter()
                stack = O.OracleStack([p], fc["w_fc"].astype(np.float64), fc["gamma_h"], wl.eps, [[K0]], [[V0]])
                prefill_s = time.perf_counter() - t0
            x, cu, H = G.round_inputs(wl, r, sched[r])
            t0 = time.perf_counter()
            outs, _ = stack.round(x, cu, H, wl.B)
            spent += time.perf_counter() - t0
            if check and done < len(gpu_outs):
                ref, got = outs[0], np.asarray(gpu_outs[done], dtype=np.float64)
                errs.append(float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)))
            done += 1
        return done, spent, prefill_s

    done, spent, prefill_s = run(budget_s, check=True)
    single = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            d1, s1, _ = run(budget_s / 3)
        single = {"value": round(d1 / s1, 3), "unit": "draft blocks/s", "threads": 1,
                  "sample": f"{d1} rounds of the cycle, {s1:.1f} s"}
    return {"value": round(done / spent, 3), "unit": "draft blocks/s", "cores": cores, "kind": "oracle",
            "blas_threads": blas, "cpu_model": _cpu_model(),
            "sample": f"{done} rounds of the {wl.rounds}-round seeded cycle (8192-row cache, 1-16 new rows, block 16), "
                      f"fp64 NumPy on {blas} BLAS threads of {cores} cores, {spent:.1f} s of round work; "
                      f"weight set-up and the oracle's prefill excluded",
            "prefill_s": round(prefill_s, 3), "single_thread": single,
            "parity": {"rounds": len(errs), "rel_l2_max": max(errs) if errs else None,
                       "rel_l2_mean": float(np.mean(errs)) if errs else None, "tolerance": 1e-2,
                       "pass": bool(errs) and max(errs) <= 1e-2,
                       "what": "the GPU's layer output of each of the cycle's first rounds (in order on a fresh "
                               "copy of the prefilled cache) against the oracle's"}}


# ---------------------------------------------------------------------------- fresh-context projections

def fresh_ctx_projections(iters):
    """MFMA utilisation of the projections on the fresh-context workload (one
    Qwen3-4B-shaped layer: d 2560, 32/8 heads of 128, k = 5 -> 12800-wide raw
    context, 1024 new context rows plus a block of 16, bf16): the layer call on
    an empty cache, timed per stage with the library's kernel-attached events.
    The fc GEMM (1024 x 12800 -> 2560) and the K/V GEMM of C (1024 x 2560 ->
    2048) run on the MFMA tile kernel; Q/K/V of the 16 block rows (one product)
    and o_proj (16 rows) stream their weights and are HBM-bound.  Beside them,
    as context, torch.matmul (hipBLASLt) on the two tile-GEMM shapes, timed the
    same way (back-to-back calls between two events)."""
    import torch

    from block_diffusion_draft_fc_amd import _lib as L
    from workloads import configs, generate as G
    from workloads.device import to_device

    wl = configs.FRESH_CTX
    dev = "cuda:0"
    n = wl.n_fixed
    fc, lw = G.fc_weights(wl), G.layer_weights(wl, 0)
    w_fc, gamma_h = to_device(fc["w_fc"], wl, dev), to_device(fc["gamma_h"], wl, dev)
    layer = L.Layer(*(to_device(lw[k], wl, dev) for k in ("w_qkv", "w_o", "gamma_q", "gamma_k")),
                    n_h=wl.n_h, n_kv=wl.n_kv, d_h=wl.d_h, eps=wl.eps, rope_theta=wl.rope_theta)
    cache = L.Cache(1, wl.n_kv, wl.d_h, torch.bfloat16, (n + wl.B + 63) // 64 * 64, device=dev)
    x, _, H = G.round_inputs(wl, 0, [n])
    xd, Hd = to_device(x, wl, dev), to_device(H, wl, dev)
    C = torch.empty((n, wl.d), dtype=torch.bfloat16, device=dev)
    out = torch.empty((wl.B, wl.d), dtype=torch.bfloat16, device=dev)
    ctx_ws = torch.empty(L.dflash_ctx_project_ws_bytes(n, wl.kd, wl.d, torch.bfloat16), dtype=torch.uint8,
                         device=dev)
    layer_ws = torch.empty(L.dflash_kv_inject_attn_ws_bytes(layer, cache, n, wl.B), dtype=torch.uint8, device=dev)

    def call():
        L.dflash_ctx_project(xd, w_fc, gamma_h, wl.eps, C, ctx_ws)
        L.dflash_kv_inject_attn(layer, cache, C, [0, n], Hd, wl.B, out, layer_ws)
        L.dflash_cache_crop(cache, [0])

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    L.timing_reset()
    head_start(iters, 300.0)
    L.timing_enable(True)
    for _ in range(iters):
        call()
    torch.cuda.synchronize()
    st = L.timing_read()
    L.timing_enable(False)
    us = {k: v[1] / max(v[0], 1) * 1e3 for k, v in st.items()}
    qd, kvd, d, kd, B = wl.n_h * wl.d_h, wl.n_kv * wl.d_h, wl.d, wl.kd, wl.B
    flops = {"ctx_gemm": 2 * n * kd * d, "qkv_gemm": 2 * (B * qd + (n + B) * 2 * kvd) * d, "o_gemm": 2 * B * qd * d}
    res = {"workload": wl.name, "iters": iters, "peak_tflops": BF16_PEAK_TFLOPS}
    for k, f in flops.items():
        t = us[k]
        res[k] = {"us": round(t, 2), "tflops": round(f / t / 1e6, 1), "mfma_frac": round(f / t / 1e6 / BF16_PEAK_TFLOPS, 4)}
    gemm_us = sum(us[k] for k in flops)
    all_us = gemm_us + us["ctx_norm"] + us["qkv_epilogue"] + us["o_reduce"]
    tot = sum(flops.values())
    res["gemms"] = {"us": round(gemm_us, 2), "tflops": round(tot / gemm_us / 1e6, 1),
                    "mfma_frac": round(tot / gemm_us / 1e6 / BF16_PEAK_TFLOPS, 4)}
    res["gemms+reductions"] = {"us": round(all_us, 2), "tflops": round(tot / all_us / 1e6, 1),
                               "mfma_frac": round(tot / all_us / 1e6 / BF16_PEAK_TFLOPS, 4)}
    res["stage_us"] = {k: round(v, 2) for k, v in us.items() if st[k][0]}
    res["vendor_matmul"] = {}
    for name, (M, K, N) in (("ctx_gemm", (n, kd, d)), ("kv_gemm_of_C", (n, d, 2 * kvd))):
        a = torch.randn((M, K), device=dev).to(torch.bfloat16)
        w = torch.randn((N, K), device=dev).to(torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, w.t())
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(iters):
            torch.matmul(a, w.t())
        ev1.record()
        torch.cuda.synchronize()
        t = ev0.elapsed_time(ev1) / iters * 1e3
        res["vendor_matmul"][name] = {"shape": f"{M} x {K} -> {N}", "us": round(t, 2),
                                      "tflops": round(2 * M * K * N / t / 1e6, 1)}
        del a, w
    return res


# ---------------------------------------------------------------------------- batched workloads

def batched_rounds(wl, rounds, ring=False):
    """Rounds of a batched workload (the 16-request ragged paged batch, or the
    5-layer hybrid stack): the seeded schedule of new context rows and the
    seeded cache lengths, with cache rows, raw context rows and block rows drawn
    on the device (values N(0,1): their statistics, not their bits, matter for
    timing).  Each round = dflash_ctx_project once + every layer's
    dflash_kv_inject_attn and crop, issued eagerly.  Three passes over the
    `rounds` scheduled rounds, the caches growing throughout: a warm-up pass,
    a timed pass and a pass with stage timing.  Reports the round time, draft
    blocks/s (one block per request per round), the attention stage's time and
    algorithmic HBM rate, and the caches' device bytes; with ring=True the
    sliding layers keep bounded ring caches."""
    import torch

    from block_diffusion_draft_fc_amd import _lib as L
    from block_diffusion_draft_fc_amd.draft_round import DraftRound
    from workloads import generate as G
    from workloads.device import to_device

    dev = "cuda:0"
    passes = 3
    g = torch.Generator(device=dev).manual_seed(wl.seed)
    L0 = G.prefill_lengths(wl)
    sched = G.schedule(wl)[:rounds]
    grow = passes * sched.sum(axis=0)
    fc = G.fc_weights(wl)
    w_fc, gamma_h = to_device(fc["w_fc"], wl, dev), to_device(fc["gamma_h"], wl, dev)
    layers, caches = [], []
    for li in range(wl.n_layers):
        lw = G.layer_weights(wl, li)
        layers.append(L.Layer(*(to_device(lw[k], wl, dev) for k in ("w_qkv", "w_o", "gamma_q", "gamma_k")),
                              n_h=wl.n_h, n_kv=wl.n_kv, d_h=wl.d_h, eps=wl.eps, rope_theta=wl.rope_theta,
                              window=wl.layer_window(li), residual=wl.n_layers > 1))
        need = [int(L0[r] + grow[r] + wl.B) for r in range(wl.R)]
        cap_ring = wl.scaled(ring=ring).ring_capacity(li)
        if cap_ring:
            caches.append(L.Cache(wl.R, wl.n_kv, wl.d_h, torch.bfloat16, cap_ring, 0, 0, dev, ring=True))
        elif wl.page_size:
            ps = wl.page_size
            caches.append(L.Cache(wl.R, wl.n_kv, wl.d_h, torch.bfloat16, sum(-(-x // ps) for x in need) + wl.R,
                                  ps, max(-(-x // ps) for x in need) + 1, dev))
        else:
            caches.append(L.Cache(wl.R, wl.n_kv, wl.d_h, torch.bfloat16, (max(need) + 63) // 64 * 64, 0, 0, dev))
    for cache in caches:
        step = cache.capacity if cache.ring else int(L0.max())
        for a in range(0, int(L0.max()), step):
            cu = [0]
            for r in range(wl.R):
                cu.append(cu[-1] + max(0, min(int(L0[r]), a + step) - a))
            k = torch.randn((cu[-1], wl.n_kv, wl.d_h), device=dev, generator=g).to(torch.bfloat16)
            v = torch.randn((cu[-1], wl.n_kv, wl.d_h), device=dev, generator=g).to(torch.bfloat16)
            L.dflash_cache_append(cache, cu, k, v)
            del k, v
    T_max = int(sched.sum(axis=1).max())
    drv = DraftRound(w_fc, gamma_h, wl.eps, layers, caches, wl.B, T_max, dev)
    xs = [torch.randn((int(sched[i].sum()), wl.kd), device=dev, generator=g).to(torch.bfloat16)
          for i in range(rounds)]
    Hs = [torch.randn((wl.R * wl.B, wl.d), device=dev, generator=g).to(torch.bfloat16) for i in range(rounds)]
    cus = [[0] + np.cumsum(sched[i]).astype(int).tolist() for i in range(rounds)]
    # algorithmic attention bytes per pass: every key a query may see, once
    att_bytes = []
    lens = [list(map(int, L0)) for _ in caches]
    for _ in range(passes):
        tot = 0
        for i in range(rounds):
            for li in range(wl.n_layers):
                W = wl.layer_window(li)
                for r in range(wl.R):
                    Lr, n = lens[li][r], int(sched[i][r])
                    lo = max(0, Lr + n - W + 1) if W else 0
                    tot += (Lr + n + wl.B - lo) * 2 * wl.n_kv * wl.d_h * 2 + wl.B * wl.n_h * wl.d_h * 2
                    lens[li][r] = Lr + n
        att_bytes.append(tot)
    torch.cuda.synchronize()

    def cycle():
        for i in range(rounds):
            drv.run(xs[i], cus[i], Hs[i])

    cycle()                      # warm-up pass
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    cycle()
    ev1.record()
    torch.cuda.synchronize()
    ms = max(ev0.elapsed_time(ev1), (time.perf_counter() - t0) * 1e3) / rounds
    L.timing_reset()
    head_start(rounds, 2000.0)
    L.timing_enable(True)
    cycle()
    torch.cuda.synchronize()
    st = L.timing_read()
    L.timing_enable(False)
    att_us = st["attn"][1] * 1e3 / rounds
    ab = att_bytes[2] / rounds
    cache_bytes = sum(c.k_pool.numel() * 2 * 2 for c in caches)
    res = {"workload": wl.name, "rounds": rounds, "requests": wl.R, "layers": wl.n_layers,
           "ring_sliding_layers": bool(ring), "ms_per_round": round(ms, 4),
           "draft_blocks_per_s": round(wl.R * 1e3 / ms, 1),
           "attn_us_per_round": round(att_us, 2), "attn_alg_bytes_per_round": int(ab),
           "attn_hbm_gbps": round(ab / (att_us * 1e-6) / 1e9, 1),
           "attn_hbm_frac": round(ab / (att_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
           "stage_us_per_round": {k: round(v[1] * 1e3 / rounds, 2) for k, v in st.items() if v[0]},
           "cache_bytes": int(cache_bytes)}
    del drv, caches, layers, xs, Hs
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------- attention at scale

def attn_pass(iters, R=4, ctx=32768, kv="bf16"):
    """The attention kernel on the Qwen3-8B head shape (32/8 heads of 128, d
    4096) for R requests with `ctx` cached keys each, 8 new context rows and a
    block of 16: every call appends its rows, attends and is cropped back, so
    each reads the same R x (ctx + 24) keys per K/V head.  R = 4, ctx = 32768
    is the full-attention layer of the 5-layer stack (537 MB in bf16); R = 1,
    ctx = 8192 the decode workload's cache.  kv "fp8" keeps the cache as E4M3
    bytes (scales 1), half the bytes.  The attention stage's time comes from
    the library's HIP events on the launch stream; K/V rows are N(0,1) drawn
    on the device (cast to E4M3 by torch for the fp8 cache)."""
    import torch

    from block_diffusion_draft_fc_amd import _lib as L
    from workloads import configs, generate as G
    from workloads.device import to_device

    wl = configs.STACK5_HYBRID
    dev = "cuda:0"
    n, B = 8, wl.B
    li = next(i for i in range(wl.n_layers) if not wl.layer_window(i))
    lw = G.layer_weights(wl, li)
    layer = L.Layer(*(to_device(lw[k], wl, dev) for k in ("w_qkv", "w_o", "gamma_q", "gamma_k")),
                    n_h=wl.n_h, n_kv=wl.n_kv, d_h=wl.d_h, eps=wl.eps, rope_theta=wl.rope_theta)
    cap = (ctx + 1024 + 63) // 64 * 64
    fp8 = kv == "fp8"
    cache = L.Cache(R, wl.n_kv, wl.d_h, torch.float8_e4m3fn if fp8 else torch.bfloat16, cap, 0, 0, dev)
    g = torch.Generator(device=dev).manual_seed(wl.seed)
    rows = []
    for _ in range(2):
        t = torch.randn((R * ctx, wl.n_kv, wl.d_h), device=dev, generator=g)
        rows.append(t.to(torch.float8_e4m3fn).view(torch.uint8) if fp8 else t.to(torch.bfloat16))
        del t
    L.dflash_cache_append(cache, [r * ctx for r in range(R + 1)], rows[0], rows[1])
    del rows
    C = torch.randn((R * n, wl.d), device=dev, generator=g).to(torch.bfloat16)
    H = torch.randn((R * B, wl.d), device=dev, generator=g).to(torch.bfloat16)
    out = torch.empty((R * B, wl.d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(L.dflash_kv_inject_attn_ws_bytes(layer, cache, R * n, B), dtype=torch.uint8, device=dev)
    cu = [r * n for r in range(R + 1)]

    def call():
        L.dflash_kv_inject_attn(layer, cache, C, cu, H, B, out, ws)
        L.dflash_cache_crop(cache, [ctx] * R)

    for _ in range(5):
        call()
    torch.cuda.synchronize()
    L.timing_reset()
    head_start(iters)
    L.timing_enable(True)
    for _ in range(iters):
        call()
    torch.cuda.synchronize()
    st = L.timing_read()
    L.timing_enable(False)
    keys = ctx + n + B
    eb = 1 if fp8 else 2
    alg = R * keys * wl.n_kv * wl.d_h * eb * 2 + R * B * wl.n_h * wl.d_h * 2
    us = st["attn"][1] * 1e3 / st["attn"][0]
    gbps = alg / (us * 1e-6) / 1e9
    res = {"shape": f"{R} requests x {keys} keys, GQA {wl.n_h}/{wl.n_kv}, d_h {wl.d_h}, block {B}, "
                    f"{'fp8 E4M3' if fp8 else 'bf16'} cache",
           "launches": st["attn"][0], "us_per_launch": round(us, 2), "alg_bytes_per_launch": int(alg),
           "gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
           "keys_per_us": round(R * keys / us, 1),
           "combine_us": round(st["attn_combine"][1] * 1e3 / st["attn_combine"][0], 2) if st["attn_combine"][0]
           else None,
           "split_merged_in_launch": st["attn_combine"][0] == 0}
    del cache, layer, C, H, out, ws
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------- acceptance

def accept_pass(iters):
    """dflash_accept on the 16-request batch (B = 16, Qwen3 vocabulary ids with
    planted match prefixes): the acceptance lengths, next-round context rows
    and anchors of a round written to device memory.  Kernel time from the
    library's stage events."""
    import torch

    from block_diffusion_draft_fc_amd import _lib as L
    from workloads import configs, generate as G

    R, B = configs.RAGGED_PAGED.R, configs.RAGGED_PAGED.B
    draft, post, _ = G.accept_tokens(configs.RAGGED_PAGED.seed, R, B, configs.QWEN3_VOCAB)
    d_draft = torch.from_numpy(draft.reshape(-1).copy()).cuda()
    d_post = torch.from_numpy(post).cuda()
    acc, rows, anchor = (torch.empty((R,), dtype=torch.int32, device="cuda") for _ in range(3))
    for _ in range(3):
        L.dflash_accept(d_draft, d_post, acc, rows, anchor)
    torch.cuda.synchronize()
    L.timing_reset()
    head_start(iters, 30.0)
    L.timing_enable(True)
    for _ in range(iters):
        L.dflash_accept(d_draft, d_post, acc, rows, anchor)
    torch.cuda.synchronize()
    st = L.timing_read()
    L.timing_enable(False)
    return {"requests": R, "block": B, "us_per_call": round(st["accept"][1] * 1e3 / st["accept"][0], 2)}


# ---------------------------------------------------------------------------- draft head

def draft_head_pass(iters):
    """The draft head after the stack ("DFlash KV Injection Walkthrough" Step
    5) for one request of the 8K decode workload: final RMSNorm of the block's
    15 tail rows, lm_head over the Qwen3 vocabulary (151936 x 4096 bf16 =
    1.24 GB, drawn on the device), argmax.  HBM-bound on the lm_head stream."""
    import torch

    from block_diffusion_draft_fc_amd import _lib as L
    from workloads import configs

    wl = configs.DECODE_8K
    vocab, d, B = configs.QWEN3_VOCAB, wl.d, wl.B
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(7)
    w = (torch.randn((vocab, d), device=dev, generator=g) / d ** 0.5).to(torch.bfloat16)
    gam = (1 + 0.1 * torch.randn((d,), device=dev, generator=g)).to(torch.bfloat16)
    h = torch.randn((B, d), device=dev, generator=g).to(torch.bfloat16)
    ids = torch.empty((B - 1,), dtype=torch.int32, device=dev)
    ws = torch.empty(L.dflash_draft_head_ws_bytes(1, B, d, vocab, torch.bfloat16), dtype=torch.uint8, device=dev)
    for _ in range(3):
        L.dflash_draft_head(h, B, gam, wl.eps, w, ids, ws)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(iters):
        L.dflash_draft_head(h, B, gam, wl.eps, w, ids, ws)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / iters
    L.timing_reset()
    head_start(iters, 50.0)
    L.timing_enable(True)
    for _ in range(iters):
        L.dflash_draft_head(h, B, gam, wl.eps, w, ids, ws)
    torch.cuda.synchronize()
    st = L.timing_read()
    L.timing_enable(False)
    gemm_us = st["head_gemm"][1] * 1e3 / iters
    alg = (vocab * d + (B - 1) * d) * 2
    res = {"workload": f"draft_head_vocab{vocab}_d{d}_rows{B - 1}_bf16", "us_per_call": round(us, 2),
           "stage_us": {k: round(v[1] * 1e3 / iters, 2) for k, v in st.items() if v[0]},
           "lm_head_alg_bytes": alg, "lm_head_gbps": round(alg / (gemm_us * 1e-6) / 1e9, 1),
           "lm_head_hbm_frac": round(alg / (gemm_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    del w
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------- device-driven rounds

def device_driven_pass(replays=3):
    """The 8K decode layer's 64-round cycle as device-driven rounds in one HIP
    graph: per round dflash_ctx_project (16 padded context rows),
    dflash_kv_inject_attn_dev (new rows from device memory), the crop back to
    the block start on the device, and dflash_accept on seeded draft/target
    tokens whose next_rows drive the next round; the graph opens by setting the
    device lengths and the first round's rows back, so every replay runs the
    same 64 rounds with no host read."""
    import torch

    from block_diffusion_draft_fc_amd import _lib as L
    from workloads import configs, generate as G
    from workloads.device import to_device

    wl = configs.DECODE_8K
    dev = "cuda:0"
    R, B, n_max, rounds, vocab = 1, wl.B, wl.B, wl.rounds, configs.QWEN3_VOCAB
    fc, lw = G.fc_weights(wl), G.layer_weights(wl, 0)
    w_fc, g_h = to_device(fc["w_fc"], wl, dev), to_device(fc["gamma_h"], wl, dev)
    layer = L.Layer(*(to_device(lw[k], wl, dev) for k in ("w_qkv", "w_o", "gamma_q", "gamma_k")),
                    n_h=wl.n_h, n_kv=wl.n_kv, d_h=wl.d_h, eps=wl.eps, rope_theta=wl.rope_theta)
    L0 = wl.prefill_len
    cap = (L0 + rounds * n_max + B + 63) // 64 * 64
    cache = L.Cache(1, wl.n_kv, wl.d_h, torch.bfloat16, cap, device=dev)
    K0, V0 = G.prefill_kv(wl, 0, 0, L0)
    L.dflash_cache_append(cache, [0, L0], to_device(np.ascontiguousarray(K0.transpose(1, 0, 2)), wl, dev),
                          to_device(np.ascontiguousarray(V0.transpose(1, 0, 2)), wl, dev))
    toks = [G.accept_tokens(wl.seed, R, B, vocab, rnd=i) for i in range(rounds)]
    n0 = int(G.schedule(wl)[0][0])
    ns = [n0] + [int(t[2][0]) + 1 for t in toks[:-1]]
    xs, Hs, drafts, posts = [], [], [], []
    for i in range(rounds):
        x, _, H = G.round_inputs(wl, i, [ns[i]])
        pad = np.zeros((n_max, wl.kd), dtype=np.float32)
        pad[:ns[i]] = x
        xs.append(to_device(pad, wl, dev))
        Hs.append(to_device(H, wl, dev))
        drafts.append(torch.from_numpy(toks[i][0].reshape(-1).copy()).to(dev))
        posts.append(torch.from_numpy(toks[i][1]).to(dev))
    C = torch.empty((n_max, wl.d), dtype=torch.bfloat16, device=dev)
    out = torch.empty((B, wl.d), dtype=torch.bfloat16, device=dev)
    cws = torch.empty(L.dflash_ctx_project_ws_bytes(n_max, wl.kd, wl.d, torch.bfloat16), dtype=torch.uint8,
                      device=dev)
    ws = torch.empty(L.dflash_kv_inject_attn_dev_ws_bytes(layer, cache, n_max, B), dtype=torch.uint8, device=dev)
    d_len = torch.zeros((1,), dtype=torch.int32, device=dev)
    d_rows = torch.zeros((1,), dtype=torch.int32, device=dev)
    rows0 = torch.tensor([n0], dtype=torch.int32, device=dev)
    acc = torch.empty((1,), dtype=torch.int32, device=dev)
    L.dflash_cache_device_begin(cache, d_len)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        L.dflash_cache_device_reset(cache, [L0])
        torch.mul(rows0, 1, out=d_rows)
        for i in range(rounds):
            L.dflash_ctx_project(xs[i], w_fc, g_h, wl.eps, C, cws)
            L.dflash_kv_inject_attn_dev(layer, cache, C, n_max, d_rows, Hs[i], B, out, ws)
            L.dflash_cache_crop_tail_dev(cache, B)
            L.dflash_accept(drafts[i], posts[i], acc, d_rows)
    g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(replays):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = max(ev0.elapsed_time(ev1), (time.perf_counter() - t0) * 1e3) / (replays * rounds)
    L.dflash_cache_device_end(cache)
    length = cache.lengths()[0]
    res = {"workload": wl.name, "rounds_per_graph": rounds, "replays": replays, "us_per_round": round(ms * 1e3, 2),
           "draft_blocks_per_s": round(1e3 / ms, 1), "final_length": int(length),
           "expected_length": int(L0 + sum(ns)), "accepted_rows_per_round": round(sum(ns) / rounds, 3)}
    del cache, layer, xs, Hs, ws
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------- profile summaries

PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_decode -o bench -- "
             "python3 -u bench.py --no-fresh-ctx --no-batched --no-cpu-baseline",
    "pmc": "rocprofv3 --pmc {c} --output-format csv -d gpurun_out/pmc_{c} -o bench -- python3 -u bench.py "
           "--no-fresh-ctx --no-batched --no-cpu-baseline --mode eager --steps 32 --warmup 4",
    "copy": "rocprofv3 --pmc {c} --output-format csv -d gpurun_out/pmc_copy_{c} -o copy -- python3 -u bench.py "
            "--copy-calibration",
}
# The 8K decode's attention launches (G3 with the split merge G4 in the same
# launch: one sequence, 8 K/V heads, one item per compute unit).
ATTN_KERNELS = ("attn_ring64_kernel<128, 4, 2, 1>",)


def attn_kernel_name(nst, d_h, merged=False):
    """The attention kernel instance the library launches for a plan's ring
    depth and head dim (bf16 layers), as rocprofv3 names it."""
    if d_h == 128:
        if nst >= 3:
            return "attn_ring64_kernel<128, 4, 2, 1>" if merged else "attn_ring64_kernel<128, 4, 2>"
        return "attn_ring64_kernel<128, 2>"
    return "attn_ring64_kernel<64, 4>"


def attn_kernel_label(L, keys, n_kv, d_h, merged):
    plan = L.dflash_attn_plan(keys, n_kv)
    name = attn_kernel_name(plan["nst"], d_h, merged)
    shape = ("two wave groups, 4-stage ring" if "4, 2" in name else
             "one wave group, 2-stage ring" if "128, 2>" in name else "one wave group")
    if merged:
        return (f"attention ({name}: split-context attention, {shape}, {plan['items']} items of "
                f"{plan['chunk']} keys, the split merged in the same launch): G3 + G4 in one launch")
    return (f"attention ({name}: split-context attention, {shape}, {plan['items']} items of "
            f"{plan['chunk']} keys) + attn_combine_kernel, the two launches of G3 + G4")


def _short(name):
    name = name.replace("void ", "")
    return name.split("(")[0]


def summarize_profiles(root):
    """Kernel-trace and HBM-counter summaries of the 8K decode bench (the
    commands in PROFILE_CMDS, run from the repository root with TMPDIR=/tmp),
    written to profiles/.  FETCH_SIZE and WRITE_SIZE are per-dispatch KiB; each
    is scaled by what it reads for a plain 256 MiB copy (262144 KiB each way)."""
    import csv
    import glob

    def rows(pattern):
        f = sorted(glob.glob(os.path.join(root, pattern)))
        if not f:
            raise SystemExit(f"no file matches {pattern} under {root}")
        return list(csv.DictReader(open(f[0])))

    stats = rows("prof_decode/*kernel_stats.csv")
    lines = ["# Kernel trace: 8K decode round (decode_ctx8k_d4096_gqa32x8_dh128_block16_bf16), one MI355X", "",
             "Command (from the repository root on the GPU box, `TMPDIR=/tmp`):", "", "```", PROFILE_CMDS["trace"],
             "```", "",
             "`bench.py` with only the headline workload: warmup, the timed steps as one graph and eagerly, "
             "then the per-stage passes (one cache, then 16 cache replicas and 2 weight sets in rotation) and "
             "the measured-peak copies and matrix product.  `mfma_peak_kernel` is mostly the register-only head "
             "start enqueued before each event-timed pass (so the host runs ahead of the GPU).  Durations are "
             "rocprofv3 kernel-trace begin/end timestamps over all calls of the command.", "",
             "| Kernel | Calls | Average µs | Min µs | Max µs | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in stats[:12]:
        lines.append(f"| `{_short(r['Name'])[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    avg = {k: next(float(r["AverageNs"]) / 1e3 for r in stats if k in r["Name"]) for k in ATTN_KERNELS}
    lines += ["", "Attention launches of the round: " + " + ".join(f"`{k}` {avg[k]:.2f} µs" for k in ATTN_KERNELS)
              + f" = {sum(avg.values()):.2f} µs on average (the split's merge runs inside the attention launch)."]
    open(os.path.join(ROOT, "profiles", "attn_decode_ctx8k_kernel_trace.md"), "w").write("\n".join(lines) + "\n")

    def per_kernel(counter, prefix):
        acc = {}
        for r in rows(f"{prefix}_{counter}/*counter_collection.csv"):
            k = _short(r["Kernel_Name"])
            a = acc.setdefault(k, [0, 0.0])
            a[0] += 1
            a[1] += float(r["Counter_Value"])
        return {k: (n, v / n) for k, (n, v) in acc.items()}

    full = 262144.0
    scale = {}
    tables = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cp = per_kernel(c, "pmc_copy")
        big = max(v for _, v in cp.values())
        scale[c] = full / big
        tables[c] = per_kernel(c, "pmc")
    lines = ["# HBM traffic counters: 8K decode round, one MI355X", "",
             "Commands (one counter per run, each its own process, from the repository root, `TMPDIR=/tmp`):",
             "", "```"] + [PROFILE_CMDS[k].format(c=c) for c in ("FETCH_SIZE", "WRITE_SIZE") for k in ("pmc", "copy")] + [
             "```", "",
             f"Calibration: a plain 256 MiB copy (262144 KiB read and written) reads FETCH_SIZE = "
             f"{full / scale['FETCH_SIZE']:.1f} KiB and WRITE_SIZE = {full / scale['WRITE_SIZE']:.1f} KiB per "
             f"dispatch, so FETCH_SIZE is scaled by {scale['FETCH_SIZE']:.3f} and WRITE_SIZE by "
             f"{scale['WRITE_SIZE']:.3f} below.", "",
             "| Kernel | Dispatches | FETCH KiB (raw) | Read MB (scaled) | WRITE KiB (raw) | Written MB (scaled) |",
             "|---|---|---|---|---|---|"]
    names = sorted(tables["FETCH_SIZE"], key=lambda k: -tables["FETCH_SIZE"][k][1] * tables["FETCH_SIZE"][k][0])
    for k in names:
        if not k.startswith(("dflash", "_ZN6dflash")):
            continue
        n, f = tables["FETCH_SIZE"][k]
        w = tables["WRITE_SIZE"].get(k, (0, 0.0))[1]
        lines.append(f"| `{k[:80]}` | {n} | {f:.1f} | {f * scale['FETCH_SIZE'] * 1024 / 1e6:.2f} | {w:.1f} | "
                     f"{w * scale['WRITE_SIZE'] * 1024 / 1e6:.2f} |")

    def bytes_of(c, key):
        k = next(k for k in tables[c] if key in k)
        return tables[c][k][1] * scale[c] * 1024

    fetch = sum(bytes_of("FETCH_SIZE", k) for k in ATTN_KERNELS)
    write = sum(bytes_of("WRITE_SIZE", k) for k in ATTN_KERNELS)
    lines += ["", "Attention of the round (" + " + ".join(f"`{k}`" for k in ATTN_KERNELS) + ") per launch: "
                  f"{fetch / 1e6:.2f} MB read + {write / 1e6:.2f} MB written = {(fetch + write) / 1e6:.2f} MB of "
                  f"HBM traffic."]
    open(os.path.join(ROOT, "profiles", "attn_decode_ctx8k_hbm_counters.md"), "w").write("\n".join(lines) + "\n")
    rec = {"kernels": list(ATTN_KERNELS), "workload": "decode_ctx8k_d4096_gqa32x8_dh128_block16_bf16",
           "attention_sources": ["block_diffusion_draft_fc_amd/csrc/" + f for f in ATTN_SOURCES],
           "attention_source_sha256": attention_source_sha256(),
           "fetch_bytes_per_launch": int(fetch), "write_bytes_per_launch": int(write),
           "fetch_scale": round(scale["FETCH_SIZE"], 4), "write_scale": round(scale["WRITE_SIZE"], 4),
           "source": "profiles/attn_decode_ctx8k_hbm_counters.md",
           "trace_us": {k: round(v, 3) for k, v in avg.items()}}
    json.dump(rec, open(os.path.join(ROOT, "profiles", "attn_decode_ctx8k_traffic.json"), "w"), indent=1)
    print(json.dumps(rec))
    return 0


# ---------------------------------------------------------------------------- measured peaks

def measured_peaks(kv_bytes):
    """The box's own figures beside the published peaks: the library's plain
    streaming read (dflash_stream_read, timed by the same kernel-attached events
    as the layer's kernels) of 1 GiB, and of the 8K round's K/V size over 17
    rotated buffers (none re-read from the 256 MB Infinity Cache: what one
    launch of that size streams from HBM); a plain 1 GiB device copy (bytes read
    + written per second); a large bf16 matrix product through torch
    (hipBLASLt); and the library's matrix-core probe (dflash_mfma_peak:
    back-to-back bf16 MFMAs on register operands, 16 waves per CU), the rate the
    matrix cores sustain at this GPU's clocks under load."""
    import torch

    from block_diffusion_draft_fc_amd import _lib as L

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, iters):
        fn(0)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(iters):
            fn(i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / iters * 1e-3

    def read_rate(bufs, iters):
        L.dflash_stream_read(bufs[0])
        torch.cuda.synchronize()
        L.timing_reset()
        L.timing_enable(True)
        for i in range(iters):
            L.dflash_stream_read(bufs[i % len(bufs)])
        torch.cuda.synchronize()
        st = L.timing_read()["stream_read"]
        L.timing_enable(False)
        return bufs[0].numel() / (st[1] * 1e-3 / st[0]) / 1e9, st[1] * 1e3 / st[0]

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    read_big, _ = read_rate([src], 10)
    dst = torch.empty_like(src)
    t = timed(lambda i: dst.copy_(src), 10)
    copy_big = 2 * n / t / 1e9
    del src, dst
    m = (kv_bytes + 255) // 256 * 256
    bufs = [torch.ones(m, dtype=torch.uint8, device="cuda") for _ in range(17)]
    read_small, us_small = read_rate(bufs, 68)
    del bufs
    a = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)
    b = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)
    t = timed(lambda i: torch.matmul(a, b), 10)
    mm = 2 * 8192 ** 3 / t / 1e12
    del a, b
    torch.cuda.empty_cache()
    iters, wgs = 4096, 1024
    L.dflash_mfma_peak(64, wgs)
    torch.cuda.synchronize()
    L.timing_reset()
    L.timing_enable(True)
    for _ in range(5):
        L.dflash_mfma_peak(iters, wgs)
    torch.cuda.synchronize()
    st = L.timing_read()["mfma_peak"]
    L.timing_enable(False)
    mfma = wgs * 4 * 8 * iters * 16384 / (st[1] * 1e-3 / st[0]) / 1e12
    return {"hbm_read_1gib_gbps": round(read_big, 1), "hbm_copy_1gib_gbps": round(copy_big, 1),
            "hbm_read_kv_size_cold_gbps": round(read_small, 1), "hbm_read_kv_size_cold_us": round(us_small, 3),
            "kv_size_bytes": int(m), "bf16_matmul_8192_tflops": round(mm, 1),
            "bf16_mfma_probe_tflops": round(mfma, 1),
            "published": {"hbm_gbps": HBM_PEAK_GBPS, "bf16_dense_tflops": BF16_PEAK_TFLOPS}}


# ---------------------------------------------------------------------------- GPU leg

def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library runs the layer on a single MI355X and "
              "implements no multi-GPU sharding.", file=sys.stderr)
        return 2

    if args.copy_calibration:
        return copy_calibration()
    if args.summarize_profiles:
        return summarize_profiles(args.summarize_profiles)
    if args.attn_pass:
        R, ctx, kv = args.attn_pass.split(",")
        if kv not in ("bf16", "fp8"):
            print("--attn-pass: KV is bf16 or fp8", file=sys.stderr)
            return 2
        print(json.dumps(attn_pass(60, int(R), int(ctx), kv)), flush=True)
        return 0

    import torch

    from block_diffusion_draft_fc_amd import _lib as L
    from workloads import configs, generate as G
    from workloads.device import to_device

    wl = configs.DECODE_8K
    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(f"bench: {wl.name}: generating weights and inputs")
    fc, lw = G.fc_weights(wl), G.layer_weights(wl, 0)

    def weight_set():
        w_fc, gamma_h = to_device(fc["w_fc"], wl, dev), to_device(fc["gamma_h"], wl, dev)
        layer = L.Layer(*(to_device(lw[k], wl, dev) for k in ("w_qkv", "w_o", "gamma_q", "gamma_k")),
                        n_h=wl.n_h, n_kv=wl.n_kv, d_h=wl.d_h, eps=wl.eps, rope_theta=wl.rope_theta)
        return w_fc, gamma_h, layer

    weights = [weight_set()]
    sched = G.schedule(wl)[:, 0]
    L0 = wl.prefill_len
    grow = int(sched.sum())
    cap = (L0 + grow + wl.B + 63) // 64 * 64
    K0, V0 = G.prefill_kv(wl, 0, 0, L0)
    # rows past the prefill (positions L0 .. L0 + grow) hold N(0,1) values too, so
    # that every round's start length (up to L0 + grow) is reachable by a crop
    K1, V1 = G.prefill_kv(wl, 0, 1, grow)
    kr = to_device(np.ascontiguousarray(np.concatenate([K0, K1], axis=1).transpose(1, 0, 2)), wl, dev)
    vr = to_device(np.ascontiguousarray(np.concatenate([V0, V1], axis=1).transpose(1, 0, 2)), wl, dev)

    def new_cache():
        c = L.Cache(1, wl.n_kv, wl.d_h, torch.bfloat16, cap, device=dev)
        L.dflash_cache_append(c, [0, L0 + grow], kr, vr)
        return c

    cache = new_cache()
    xs, Hs = [], []
    for rnd in range(wl.rounds):
        x, _, H = G.round_inputs(wl, rnd, [int(sched[rnd])])
        xs.append(to_device(x, wl, dev))
        Hs.append(to_device(H, wl, dev))
    max_n = int(sched.max())
    C = torch.empty((max_n, wl.d), dtype=torch.bfloat16, device=dev)
    out = torch.empty((wl.B, wl.d), dtype=torch.bfloat16, device=dev)
    ctx_ws = torch.empty(L.dflash_ctx_project_ws_bytes(max_n, wl.kd, wl.d, torch.bfloat16), dtype=torch.uint8,
                         device=dev)
    layer_ws = torch.empty(L.dflash_kv_inject_attn_ws_bytes(weights[0][2], cache, max_n, wl.B),
                           dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # cache length at the start of round r of a 64-round cycle
    starts = L0 + np.concatenate([[0], np.cumsum(sched)[:-1]])

    def step(i, c=None, w=None):
        """Round i % 64 on cache c with weight set w: crop back to the round's
        start, fc + hidden_norm, the layer, crop to the accepted prefix."""
        c = cache if c is None else c
        w_fc, gamma_h, layer = weights[0] if w is None else w
        r = i % wl.rounds
        cur, st0 = c.lengths()[0], int(starts[r])
        if cur < st0:
            # a cold replica last ran an earlier round: bring it up to this
            # round's start with the same rows the cache held there
            L.dflash_cache_append(c, [0, st0 - cur], kr[cur:st0], vr[cur:st0])
        L.dflash_cache_crop(c, [st0])
        n = int(sched[r])
        Cn = C[:n]
        L.dflash_ctx_project(xs[r], w_fc, gamma_h, wl.eps, Cn, ctx_ws)
        L.dflash_kv_inject_attn(layer, c, Cn, [0, n], Hs[r], wl.B, out, layer_ws)
        L.dflash_cache_crop(c, [st0 + n])

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(run):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record()
        run()
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return max(ev0.elapsed_time(ev1), wall * 1e3) / args.steps

    # W untimed warmup steps (rounds 0 .. W-1), then the K timed steps (rounds
    # W .. W+K-1 of the cycle), eagerly and as one HIP graph of exactly those K
    # steps.  Capture runs the library's host side (validation, planning, cache
    # metadata) and records the kernels with their arguments; every round crops
    # back to its own start first, so a replay rewrites the rows it wrote at
    # capture and the cache metadata the capture left stays valid.
    first = args.warmup
    for i in range(args.warmup):
        step(i)
    eager_ms = graph_ms = None
    if args.mode in ("eager", "best"):
        eager_ms = timed(lambda: [step(first + i) for i in range(args.steps)])
    if args.mode in ("graph", "best"):
        log(f"bench: capturing the {args.steps} timed steps as one graph")
        s = torch.cuda.Stream()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(args.steps):
                step(first + i)
        g.replay()
        graph_ms = timed(g.replay)
    if args.mode == "graph" or (args.mode == "best" and graph_ms <= eager_ms):
        ms_per_step, mode = graph_ms, "graph"
    else:
        ms_per_step, mode = eager_ms, "eager"
    fmt = lambda ms: "-" if ms is None else f"{ms * 1e3:.1f}"  # noqa: E731
    log(f"bench: graph {fmt(graph_ms)} us/step, eager {fmt(eager_ms)} us/step -> {mode}")

    # ---------------- per-stage times from the library's kernel-attached HIP
    # events on the launch stream, over the same K rounds issued eagerly.
    #  warm: one cache and one weight set, as in the timed steps;
    #  cold: 16 cache replicas (each 36 MB, 16 x 36 MB > 512 MB) and 2 weight
    #  sets in rotation, so no kernel finds its K/V or weights among the last
    #  256 MB of traffic (the size of the Infinity Cache): the attention reads
    #  its K/V from HBM.
    def stage_pass(pick):
        L.timing_reset()
        head_start(args.steps)
        L.timing_enable(True)
        for i in range(args.steps):
            step(first + i, *pick(i))
        torch.cuda.synchronize()
        st = L.timing_read()
        L.timing_enable(False)
        return st

    stages_warm = stage_pass(lambda i: (None, None))
    log("bench: cold protocol (16 cache replicas, 2 weight sets)")
    replicas = [new_cache() for _ in range(16)]
    weights.append(weight_set())
    torch.cuda.synchronize()
    stages = stage_pass(lambda i: (replicas[i % 16], weights[i % 2]))
    replica_bytes = sum(c.k_pool.numel() * 2 * 2 for c in replicas)
    del replicas
    weights.pop()
    torch.cuda.empty_cache()

    # algorithmic work of the timed steps
    work = {}
    for i in range(args.steps):
        r = (first + i) % wl.rounds
        for k, v in round_work(wl, int(starts[r]), int(sched[r])).items():
            a = work.setdefault(k, {"bytes": 0, "flops": 0})
            a["bytes"] += v["bytes"]
            a["flops"] += v["flops"]

    def stage_entry(st, name, stage_names, bound):
        n = st[stage_names[0]][0]
        ms = sum(st[x][1] for x in stage_names)
        us = ms / max(n, 1) * 1e3
        b, f = work[name]["bytes"] / max(n, 1), work[name]["flops"] / max(n, 1)
        gbps = b / (us * 1e-6) / 1e9 if us > 0 else 0.0
        tflops = f / (us * 1e-6) / 1e12 if us > 0 else 0.0
        return {"stages": list(stage_names), "launches": n, "us_per_launch": round(us, 3),
                "alg_bytes_per_launch": int(b), "alg_flops_per_launch": int(f),
                "gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
                "tflops": round(tflops, 2), "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 5), "bound": bound}

    def kernel_table(st):
        return {
            "attn+combine": stage_entry(st, "attn", ["attn", "attn_combine"], "hbm"),
            "attn": stage_entry(st, "attn", ["attn"], "hbm"),
            "ctx_project": stage_entry(st, "ctx_gemm", ["ctx_gemm", "ctx_reduce", "ctx_norm"], "hbm"),
            "ctx_gemm_only": stage_entry(st, "ctx_gemm", ["ctx_gemm"], "hbm"),
            "qkv": stage_entry(st, "qkv_gemm", ["qkv_gemm", "qkv_epilogue"], "hbm"),
            "o_proj": stage_entry(st, "o_gemm", ["o_gemm", "o_reduce"], "hbm"),
        }

    kernels, kernels_warm = kernel_table(stages), kernel_table(stages_warm)
    stage_us = {k: round(v[1] / max(v[0], 1) * 1e3, 3) for k, v in stages.items() if v[0]}
    stage_us_warm = {k: round(v[1] / max(v[0], 1) * 1e3, 3) for k, v in stages_warm.items() if v[0]}
    peaks = measured_peaks(work["attn"]["bytes"] // args.steps)

    att = kernels["attn+combine"]
    round_bytes = work["round"]["bytes"] / args.steps
    blocks_per_s = 1e3 / ms_per_step
    res = {
        "metric": METRIC,
        "value": round(blocks_per_s, 1),
        "unit": "draft blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "graph_ms_per_step": graph_ms and round(graph_ms, 5),
        "eager_ms_per_step": eager_ms and round(eager_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, N(0,1/fan_in) weights)",
        "config": {"workload": wl.name, "ctx": L0, "block": wl.B, "heads": f"{wl.n_h}/{wl.n_kv}", "d": wl.d,
                   "d_h": wl.d_h, "k_layers": wl.k_layers, "rounds_per_cycle": wl.rounds, "batch": wl.R,
                   "mode": mode},
        "attn_hbm_gbps": att["gbps"],
        "attn_hbm_frac_peak": att["hbm_frac"],
        "roofline": {"bound": "hbm", "achieved": att["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": att["hbm_frac"], "traffic": traffic_record(),
                     "kernel": attn_kernel_label(L, [L0 + wl.B + 8] * wl.R, wl.n_kv, wl.d_h,
                                                 stages["attn_combine"][0] == 0),
                     "protocol": "cold: 16 cache replicas and 2 weight sets in rotation",
                     "us_per_launch": att["us_per_launch"], "alg_bytes_per_launch": att["alg_bytes_per_launch"],
                     "attn_us": kernels["attn"]["us_per_launch"],
                     "combine_us": round(att["us_per_launch"] - kernels["attn"]["us_per_launch"], 3),
                     "frac_of_measured_read_peak": round(att["gbps"] / peaks["hbm_read_1gib_gbps"], 4),
                     "frac_of_same_size_read": round(att["gbps"] / peaks["hbm_read_kv_size_cold_gbps"], 4),
                     "warm": {"achieved": kernels_warm["attn+combine"]["gbps"],
                              "frac": kernels_warm["attn+combine"]["hbm_frac"],
                              "us_per_launch": kernels_warm["attn+combine"]["us_per_launch"],
                              "attn_us": kernels_warm["attn"]["us_per_launch"]}},
        "measured_peaks": peaks,
        "round_alg_bytes": int(round_bytes),
        "round_hbm_gbps": round(round_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "kernels": kernels,
        "kernels_warm": kernels_warm,
        "stage_us": stage_us,
        "stage_us_warm": stage_us_warm,
        "cold_replica_bytes": int(replica_bytes),
    }
    if not args.no_fresh_ctx:
        log("bench: fresh-context projections")
        fc = fresh_ctx_projections(20)
        # the same rates against what the matrix cores sustain on this GPU
        probe = peaks["bf16_mfma_probe_tflops"]
        fc["mfma_probe_tflops"] = probe
        for k in ("ctx_gemm", "qkv_gemm", "gemms"):
            fc[k]["frac_of_mfma_probe"] = round(fc[k]["tflops"] / probe, 4)
        res["fresh_ctx_projections"] = fc
    if not args.no_batched:
        log("bench: attention kernel on the stack's full-attention layer shape")
        res["attn_at_scale"] = attn_pass(30, 4, 32768, "bf16")
        log("bench: attention over fp8 caches")
        res["fp8_kv_cache"] = {"ctx8k_batch1": attn_pass(60, 1, 8192, "fp8"),
                               "ctx8k_batch1_bf16_same_harness": attn_pass(60, 1, 8192, "bf16"),
                               "ctx32k_batch4": attn_pass(30, 4, 32768, "fp8")}
        log("bench: draft head (lm_head over the Qwen3 vocabulary)")
        res["draft_head"] = draft_head_pass(20)
        log("bench: acceptance of a 16-request round")
        res["accept"] = accept_pass(100)
        log("bench: device-driven rounds (64 in one graph, acceptance on the device)")
        res["device_driven_graph"] = device_driven_pass()
        log("bench: ragged 16-request paged batch")
        res["ragged_paged"] = batched_rounds(configs.RAGGED_PAGED, 16)
        log("bench: 5-layer hybrid stack, ring caches on the sliding layers")
        res["stack5_hybrid_ring"] = batched_rounds(configs.STACK5_HYBRID, 8, ring=True)
        log("bench: 5-layer hybrid stack, unbounded caches")
        res["stack5_hybrid_full_caches"] = batched_rounds(configs.STACK5_HYBRID, 8, ring=False)
    if not args.no_cpu_baseline:
        # rounds 0 .. PARITY_ROUNDS - 1 in order on a fresh copy of the prefilled
        # cache: the outputs the CPU leg sets against the oracle's
        log("bench: the cycle's first rounds in order, for the parity check")
        pc = new_cache()
        L.dflash_cache_crop(pc, [L0])
        par_outs = []
        for r in range(PARITY_ROUNDS):
            step(r, pc)
            par_outs.append(out.float().cpu().numpy())
        del pc
        torch.cuda.empty_cache()
        log("bench: timing the fp64 oracle on the host")
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, par_outs)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
