#!/usr/bin/env python3
"""Benchmark of the per-hop KV-cache correction (KVCMAS hot path) on one MI355X.

Workload (one step = one whole hop): a Llama-3.1-8B-shaped shared segment of 32768 tokens,
32 layers, 8 KV heads x 128 (D = 1024 per K and per V), bf16, corrected against a pool of
20 anchors stored as rank-32 factors; shift 300 positions; one third of the layers carry a
source no anchor holds.  Every step re-aligns, scores, gates, weights and applies the delta
for all layers, keys and values, through kvc_correct_hop.  Inputs are synthetic (seeded
generator) and resident in HBM before the timed region.

Prints one JSON line: corrected KV tokens/s (all layers), the roofline of the dominant kernel
(measured with HIP events around each launch on the library's stream) and the fp64 CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "corrected KV tokens/s (all layers) at 8B shape, 32K seg; % HBM/MFMA roofline"
PEAK_HBM = 8.0e12            # B/s, MI355X HBM3E
PEAK_MFMA_BF16 = 2.5e15      # flop/s, dense bf16
# VALU lane-ops/s: the published fp32 vector peak, 157.3 TFLOP/s with an FMA counted as 2, is
# 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz = 78.6 T lane-ops/s.  Plain (unpacked) v_add_f32
# reaches it too: the library's VALU loop sustains ~62 T lane-ops/s on the device, above what
# a 16-lane SIMD could issue at any clock it runs.
PEAK_VALU_OPS = 256 * 4 * 32 * 2.4e9


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_work(name, L, S, D, N, rC, rD, mode="pages", b=2):
    """Algorithmic HBM bytes, MFMA flops and VALU lane-ops of one launch of `name` (whole hop).

    Bytes count each operand once: the K/V source read, the corrected K/V written, the A and B
    factors the launch contracts (B in its packed operand form, same size), the fp32 scores a
    second-mode launch reads.  Flops are the MFMA contractions (2 per multiply-add).  VALU
    lane-ops are the first-mode epilogue: one |E| add per (token, channel, anchor) on both sides
    plus one E^2 fma on the value side."""
    src = 2 * L * S * D * b                       # K and V source read
    out = 2 * L * S * D * b                       # corrected K and V written
    fac_base = 2 * L * N * (S * rC + D * rC) * b  # base A and B, both sides
    fac_delta = 2 * L * N * (S * rD + D * rD) * b
    scores = 2 * L * S * N * 4
    if name == "fused_hop" and mode == "pages":
        return dict(bytes=src + out + fac_base + fac_delta, flops=4 * L * S * D * N * (rC + rD), alu=3 * L * S * D * N)
    if name == "fused_hop":                       # second mode: weights from materialised scores
        return dict(bytes=src + out + fac_delta + scores, flops=4 * L * S * D * N * rD, alu=0)
    if name == "split_score":                     # first mode: per-token distances + gate sums
        return dict(bytes=src + fac_base + scores, flops=4 * L * S * D * N * rC, alu=3 * L * S * D * N)
    if name == "split_apply":                     # token weights from the scores, then the delta
        return dict(bytes=src + out + fac_delta + scores, flops=4 * L * S * D * N * rD, alu=0)
    if name in ("score_cos_mfma", "score_cos_gemm"):
        return dict(bytes=src + fac_base + scores, flops=4 * L * S * D * N * rC, alu=6 * L * S * N * rC)
    if name == "split_weights":                   # per-channel-tile distance partials in, weights out
        return dict(bytes=2 * L * S * N * 4 * (D // 256 + 1), flops=0, alu=0)
    if name in ("pack_base", "pack_delta", "pack_cos"):
        r = rD if name == "pack_delta" else rC
        return dict(bytes=2 * 2 * L * N * r * D * b, flops=0, alu=0)
    return dict(bytes=0, flops=0, alu=0)


def roofline(name, ms, work, traffic=None):
    t = ms / 1e3
    cands = [("hbm", work["bytes"] / PEAK_HBM, work["bytes"] / t / 1e9, PEAK_HBM / 1e9, "GB/s"),
             ("mfma", work["flops"] / PEAK_MFMA_BF16, work["flops"] / t / 1e12, PEAK_MFMA_BF16 / 1e12, "TFLOP/s"),
             ("alu", work["alu"] / PEAK_VALU_OPS, work["alu"] / t / 1e12, PEAK_VALU_OPS / 1e12, "Tops/s")]
    bound, _, ach, peak, unit = max(cands, key=lambda c: c[1])
    return {"kernel": name, "bound": bound, "achieved": round(ach, 3), "peak": round(peak, 3), "unit": unit,
            "frac": round(ach / peak, 4), "traffic": traffic, "ms": round(ms, 4),
            "algorithmic_bytes": work["bytes"], "mfma_flops": work["flops"], "valu_ops": work["alu"]}


def measured_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on this kernel's
    current source."""
    from rank_kv_cache_layer_amd.profsum import kernel_source_hash
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    v = d.get("kernels", {}).get(kernel)
    if not isinstance(v, dict) or v.get("source_hash") != kernel_source_hash(kernel):
        return None
    return int(v["bytes"])


def measure_peaks(kvc, torch):
    """Device ceilings from the library's measurement kernels, timed with events on the stream
    they run on: HBM copy (read + write bytes), bf16 MFMA, LDS reads, unpacked fp32 VALU."""
    st = torch.cuda.current_stream()

    def timed(fn, reps):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    nb = 1 << 30
    a = torch.empty(nb, dtype=torch.uint8, device="cuda")
    b = torch.empty(nb, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    t_copy = timed(lambda: kvc.peak_copy(b, a), 10)
    del a, b
    blocks = 256 * 8
    it_m, it_l, it_v = 64, 8192, 65536     # about 7-30 ms per launch at the published peaks
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    t_mfma = timed(lambda: kvc.peak_loop("mfma", sink, blocks, it_m), 3)
    t_lds = timed(lambda: kvc.peak_loop("lds", sink, blocks, it_l), 3)
    t_valu = timed(lambda: kvc.peak_loop("valu", sink, blocks, it_v), 3)
    return {"hbm_copy_GBps": round(2 * nb / t_copy / 1e9, 1),
            "mfma_bf16_TFLOPs": round(blocks * 4 * it_m * 4 * 32768 / t_mfma / 1e12, 1),
            "lds_read_bytes_per_clk_per_CU_at_2.4GHz": round(blocks * 256 * it_l * 8 * 16 / t_lds / 256 / 2.4e9, 1),
            "valu_fp32_Tops": round(blocks * 256 * it_v * 8 / t_valu / 1e12, 2)}


def measure_refresh(kvc, torch, n_mats=64, rows=4096, cols=1024, rank=128, p=32, q=3, reps=3, oracle=True):
    """Anchor refresh at its configuration: 32 layers x (K, V) fp32 deltas of 4096 x 1024 with a
    decaying spectrum, rank 128 (oversample 32, 3 power iterations).  Inputs are generated on
    the device (Gaussian factors with i^-1.5 column scales), resident before timing."""
    g = torch.Generator(device="cuda").manual_seed(3)
    sc = torch.arange(1, cols + 1, device="cuda", dtype=torch.float32) ** -1.5
    z = torch.empty((n_mats, rows, cols), device="cuda")
    for m in range(n_mats):
        a = torch.randn((rows, cols), device="cuda", generator=g) * sc[None, :]
        z[m] = a @ (torch.randn((cols, cols), device="cuda", generator=g) / cols ** 0.5)
    ws = torch.empty((kvc.svd_workspace_size(n_mats, rows, cols, rank, p),), dtype=torch.uint8, device="cuda")
    kvc.anchor_refresh_svd(z, rank, oversample=p, power_iters=q, workspace=ws)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        kvc.anchor_refresh_svd(z, rank, oversample=p, power_iters=q, workspace=ws)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    l = rank + p
    flops = n_mats * 2.0 * rows * cols * l * (2 * q + 2)          # sketch, power iterations, Q^T Z
    out = {"workload": f"{n_mats} x {rows}x{cols} fp32, rank {rank}, oversample {p}, {q} power iterations",
           "ms": round(ms, 3), "matrices_per_s": round(n_mats / (ms / 1e3), 1),
           "gemm_flops": int(flops), "achieved_TFLOPs": round(flops / (ms / 1e3) / 1e12, 2),
           "peak_fp32_vector_TFLOPs": 157.3}
    if oracle:
        # the oracle's factorisation (exact fp64 SVD) of one of the same matrices
        from oracle import kvc_oracle as O
        zm = z[0].double().cpu().numpy()
        t0 = time.perf_counter()
        O.truncated_svd(zm, rank)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(1.0 / dt, 3), "unit": "matrices/s", "kind": "oracle",
                               "sample": f"1 of the {n_mats} matrices, fp64 SVD, {dt:.2f} s"}
    return out


def measure_pool_insert(kvc, torch, L=32, S=4096, H=8, hd=128, r=32, V=20, p=16, q=2, reps=3, oracle=True):
    """One pool update after a dense fallback (App. A.3 "Cache Materialization and Pool Updates":
    Eq. 12, then Eq. 7 factorisation) at the 8B shape on a 4096-token segment: canonical source
    and observed correction of K and V, each factorised at rank 32 (oversample 16, 2 power
    iterations) and written into slot 7 of a 20-slot bf16 arena.  Also the Eq. 12 kernels alone
    (HBM-bound: algorithmically 4 bf16 reads and 4 fp32 writes of L x S x D; the sources are read
    once for the base and once for the correction).  Inputs generated on the device, resident
    before timing."""
    D = H * hd
    g = torch.Generator(device="cuda").manual_seed(7)
    ks, vs, kt, vt = (torch.randn((L, S, D), device="cuda", generator=g).to(torch.bfloat16) for _ in range(4))
    zt = lambda *sh: torch.zeros(sh, dtype=torch.bfloat16, device="cuda")
    arena = kvc.PoolTensors(anchor_len=[0] * V, rank_base=r, rank_delta=r, baseA_k=zt(L, V * S, r),
                            baseB_k=zt(L, V, r, D), baseA_v=zt(L, V * S, r), baseB_v=zt(L, V, r, D),
                            deltaA_k=zt(L, V * S, r), deltaB_k=zt(L, V, r, D), deltaA_v=zt(L, V * S, r),
                            deltaB_v=zt(L, V, r, D), slot_rows=S, live=[0] * V)
    shp = kvc.shape_of(L, S, H, hd)
    ws = torch.empty((kvc.pool_insert_workspace(shp, arena, p),), dtype=torch.uint8, device="cuda")
    ins = lambda: kvc.pool_insert(ks, vs, kt, vt, shp, 512, 812, arena, 7, oversample=p, power_iters=q, seed=1,
                                  workspace=ws)
    outs = [torch.empty((L, S, D), device="cuda") for _ in range(4)]
    delta = lambda: kvc.observed_delta(ks, vs, kt, vt, shp, 512, 812, *outs)

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(n):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms = timed(ins, reps)
    ms_d = timed(delta, 10)
    nbytes = L * S * D * (4 * 2 + 4 * 4)   # each cache read once, four fp32 results written
    out = {"workload": f"one fallback insert, {L} layers x {S} tokens x {H}x{hd} bf16, K and V, rank {r} "
                       f"(oversample {p}, {q} power iterations), arena of {V} slots",
           "ms": round(ms, 3), "inserts_per_s": round(1e3 / ms, 2),
           "eq12_kernels": {"ms": round(ms_d, 4), "bound": "hbm", "algorithmic_bytes": nbytes,
                            "achieved_GBps": round(nbytes / (ms_d / 1e3) / 1e9, 1), "peak_GBps": 8000.0,
                            "frac": round(nbytes / (ms_d / 1e3) / 8e12, 4)}}
    if oracle:
        # the oracle on one layer's keys (canonical source + Eq. 12 + two fp64 factorisations),
        # scaled to both sides and all layers
        from oracle import kvc_oracle as O
        a, b = ks[0].double().cpu().numpy(), kt[0].double().cpu().numpy()
        t0 = time.perf_counter()
        fr = O.inv_freq(hd)
        O.truncated_svd(O.rope(a, -512, hd, fr), r)
        O.truncated_svd(O.observed_delta(b, a, 512, 812, hd, True), r)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(1.0 / (dt * 2 * L), 4), "unit": "inserts/s", "kind": "oracle",
                               "sample": f"layer 0 keys: Eq. 12 + 2 fp64 SVDs of {S}x{D}, {dt:.2f} s, "
                                         f"scaled to {2 * L} layer-sides"}
    del ks, vs, kt, vt, arena, ws, outs
    torch.cuda.empty_cache()
    return out


def measure_rank128(kvc, torch, W, data, steps=5):
    """Rank-128 correction (32 layers x 4096 tokens x 8x128 bf16, 10 anchors at rank 128 for base
    and delta), both scoring modes, through the library's default path for that rank."""
    sp = data.spec
    k, v = data.k_src.to("cuda"), data.v_src.to("cuda")
    ko, vo = torch.empty_like(k), torch.empty_like(v)
    pool = kvc.pool_from(data, "cuda")
    shp = kvc.shape_of(sp.n_layers, sp.seq_len, sp.n_kv_heads, sp.head_dim)
    L, S, D, N, r = sp.n_layers, sp.seq_len, sp.d_model, sp.n_anchors, sp.rank_base
    flops = 4 * L * S * D * N * (r + sp.rank_delta)
    nbytes = 2 * L * S * D * (2 + 2) + 2 * L * N * (r + sp.rank_delta) * (S + D) * 2
    out = {"workload": f"{L} layers x {S} tokens x {sp.n_kv_heads}x{sp.head_dim} bf16, {N} anchors at rank {r}",
           "mfma_flops": flops, "algorithmic_bytes": nbytes}
    for name, mode in (("pages", W.SCORE_PAGES), ("cos_r", W.SCORE_COS_R)):
        prm_fn = lambda tr, m=mode: kvc.params_of(sp.tau, sp.temp_gate, sp.temp_weight, sp.gate_len, m, 0, tr)
        ws = torch.empty((kvc.correct_hop_workspace(shp, pool, prm_fn(None)),), dtype=torch.uint8, device="cuda")
        ms, _, per_kernel, _ = time_hop(kvc, torch, k, v, ko, vo, shp, sp, pool, prm_fn, ws, steps, 2)
        out[name] = {"ms": round(ms, 4), "tokens_per_s": round(S / (ms / 1e3), 1),
                     "mfma_frac": round(flops / (ms / 1e3) / PEAK_MFMA_BF16, 4),
                     "kernels_ms": {n: round(statistics.median(t), 4) for n, t in per_kernel.items()}}
    return out


def measure_pf_delta(kvc, torch, L=32, S=32768, H=8, hd=128, r=8, reps=10):
    """App. A.2: a recurring relation's correction, profiled once and stored at rank 8, reused
    with weight 1 and re-alignment and no matching (kvc_apply_lowrank_delta with one anchor),
    at the 32K-token 8B shape.  HBM-bound: source and output of K and V, the rank-8 factors and
    the given weights.  Inputs generated on the device, resident before timing."""
    D = H * hd
    g = torch.Generator(device="cuda").manual_seed(9)
    k, v = (torch.randn((L, S, D), device="cuda", generator=g).to(torch.bfloat16) for _ in range(2))
    mk = lambda *sh: (torch.randn(sh, device="cuda", generator=g) * 0.1).to(torch.bfloat16)
    pool = kvc.PoolTensors([S], 16, r, mk(L, S, 16), mk(L, 1, 16, D), mk(L, S, 16), mk(L, 1, 16, D),
                           mk(L, S, r), mk(L, 1, r, D), mk(L, S, r), mk(L, 1, r, D))
    w = torch.ones((L, S, 1), dtype=torch.float32, device="cuda")
    ko, vo = torch.empty_like(k), torch.empty_like(v)
    shp = kvc.shape_of(L, S, H, hd)
    ws = torch.empty((max(kvc.workspace_size(kvc.CALL_APPLY, shp, pool), 16),), dtype=torch.uint8, device="cuda")
    run = lambda tr=None: kvc.apply_lowrank_delta(k, v, ko, vo, shp, 512, 812, pool, w, w, S, workspace=ws)
    run()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        run()
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = 2 * L * S * D * 2 * 2 + 2 * L * (S * r + r * D) * 2 + 2 * L * S * 4
    out = {"workload": f"rank-{r} correction with weight 1 (no matching), {L} layers x {S} tokens x {H}x{hd} bf16",
           "ms": round(ms, 4), "tokens_per_s": round(S / (ms / 1e3), 1), "bound": "hbm",
           "algorithmic_bytes": nbytes, "achieved_GBps": round(nbytes / (ms / 1e3) / 1e9, 1), "peak_GBps": 8000.0,
           "frac": round(nbytes / (ms / 1e3) / 8e12, 4)}
    del k, v, ko, vo, pool, w, ws
    torch.cuda.empty_cache()
    return out


def measure_study(torch, L=8, S=4096, D=1024, rank=32):
    """Sec. 3.2 / Fig. 3(b) analogue on synthetic exact caches (each agent adds a rank-24
    deviation with 1% full-rank noise to the trajectory so far): per-agent normalised error of
    chained (Eq. 6, exact first agent) and reference-based (Eq. 4) correction at rank 32, run with
    the library's factorisation and apply."""
    from rank_kv_cache_layer_amd import study
    from rank_kv_cache_layer_amd import workload as W
    ref, agents = W.chain_study_caches(n_layers=L, seq_len=S, d=D, device="cuda")
    t0 = time.perf_counter()
    res = study.chain_vs_reference(ref, agents, rank)
    dt = time.perf_counter() - t0
    del ref, agents
    torch.cuda.empty_cache()
    return {"workload": f"4 agents A0 -> A3, {L} layers x {S} x {D} fp32, per-agent deviation rank 24 + 1% noise, "
                        f"correction rank {rank}",
            "error_chained": [round(x, 5) for x in res["chained"]],
            "error_non_chained": [round(x, 5) for x in res["non_chained"]], "wall_s": round(dt, 3)}


def measure_chain(kvc, torch, W, n_requests=8, n_hops=3, steps=3):
    """Concurrent chains (A0 -> A1 -> A2 -> A3) at the 8B shape, 8192 tokens per request: the
    seeded chain specification (per hop 10-20 anchors, rank 16 or 32, positions) with factors and
    first sources drawn on the device (N(0, 1) sources, factors N(0, 0.2^2), bf16), since the
    time does not depend on the values; all requests' hops in one kvc_correct_hops_batched
    call.  Tokens/s counts every hop's corrected segment."""
    reqs = W.chain_specs(n_requests=n_requests, n_hops=n_hops)
    h0 = reqs[0][0]
    L, S, D = h0.n_layers, h0.seq_len, h0.n_kv_heads * h0.head_dim
    shp = kvc.shape_of(L, S, h0.n_kv_heads, h0.head_dim)
    g = torch.Generator(device="cuda").manual_seed(4)
    rnd = lambda *sh, sc=1.0: (torch.randn(sh, device="cuda", generator=g) * sc).to(torch.bfloat16)
    hl = []
    for hops in reqs:
        base = len(hl)
        k0, v0 = rnd(L, S, D), rnd(L, S, D)
        for i, h in enumerate(hops):
            N, r = h.n_anchors, h.rank_base
            f = lambda rr: (rnd(L, N * S, rr, sc=0.2), rnd(L, N, rr, D, sc=0.2))
            (bAk, bBk), (bAv, bBv), (dAk, dBk), (dAv, dBv) = f(r), f(r), f(h.rank_delta), f(h.rank_delta)
            pool = kvc.PoolTensors([S] * N, r, h.rank_delta, bAk, bBk, bAv, bBv, dAk, dBk, dAv, dBv)
            out = kvc.alloc_match(L, S, N, "cuda", want_weights=False)
            hl.append(kvc.Hop(k0 if i == 0 else None, v0 if i == 0 else None, torch.empty_like(k0),
                              torch.empty_like(v0), h.p_src, h.p_tgt, base + i - 1 if i else -1, pool, out))
    prm = kvc.params_of(h0.tau, h0.temp_gate, h0.temp_weight, h0.gate_len, h0.mode, 0, None)
    ws = torch.empty((kvc.hops_batched_workspace(hl, shp, prm),), dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream()

    def timed(one):
        kvc.correct_hops_batched(hl, shp, prm, workspace=ws, one_at_a_time=one)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(steps):
            kvc.correct_hops_batched(hl, shp, prm, workspace=ws, one_at_a_time=one)
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(False)
    ms_one = timed(True)
    tr = kvc.KernelTrace(32)
    kvc.correct_hops_batched(hl, shp, kvc.params_of(h0.tau, h0.temp_gate, h0.temp_weight, h0.gate_len, h0.mode, 0, tr),
                             workspace=ws)
    torch.cuda.synchronize()
    per_kernel = {}
    for name, t in tr.results():
        per_kernel[name] = per_kernel.get(name, 0.0) + t
    tr.close()
    toks = sum(h.seq_len for hops in reqs for h in hops)
    nbytes = sum(int(t.numel()) * 2 for h in hl for t in (h.k_out, h.v_out))
    nbytes += sum(int(t.numel()) * 2 for h in hl if h.k_src is not None for t in (h.k_src, h.v_src))
    nbytes += sum(int(t.numel()) * 2 for h in hl for t in (h.pool.baseA_k, h.pool.baseB_k, h.pool.baseA_v,
                                                            h.pool.baseB_v, h.pool.deltaA_k, h.pool.deltaB_k,
                                                            h.pool.deltaA_v, h.pool.deltaB_v))
    flops = sum(4 * L * S * D * h.n_anchors * (h.rank_base + h.rank_delta) for hops in reqs for h in hops)
    floor_ms = max(nbytes / PEAK_HBM, flops / PEAK_MFMA_BF16) * 1e3
    out = {"workload": f"{n_requests} requests x {n_hops} chained hops, {L} layers x {S} tokens, "
                       f"{h0.n_kv_heads}x{h0.head_dim} KV heads, bf16, pools of 10-20 anchors at rank 16/32 "
                       f"(seeded chain specification, values drawn on the device); each chain level one grid "
                       f"per kernel",
           "ms": round(ms, 3), "tokens_per_s": round(toks / (ms / 1e3), 1),
           "ms_one_hop_per_call": round(ms_one, 3),
           "algorithmic_bytes": nbytes, "mfma_flops": flops, "achieved_GBps": round(nbytes / (ms / 1e3) / 1e9, 1),
           "achieved_TFLOPs": round(flops / (ms / 1e3) / 1e12, 1), "roofline_floor_ms": round(floor_ms, 3),
           "frac_of_floor": round(floor_ms / ms, 4),
           "kernels_ms_per_batch": {n: round(t, 4) for n, t in per_kernel.items()}}
    del hl, ws
    torch.cuda.empty_cache()
    return out


def host_info():
    """The host the oracle runs on: CPU model, logical CPUs, BLAS threads."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas = 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:
        affinity = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "sched_affinity": affinity, "blas_threads": int(blas)}


def _layers_of(data, layers, **repl):
    """The hop's inputs restricted to `layers` (the oracle then sees layer i of the list as layer i)."""
    import torch
    idx = torch.tensor(layers)
    t = {k: v.index_select(0, idx) for k, v in data.tensors().items()}
    t.update(repl)
    return dataclasses.replace(data, spec=dataclasses.replace(data.spec, n_layers=len(layers)), **t)


def hop_quality(O, W, data, gpu, layers, exact=True):
    """Parity and correction quality on sampled layers, all tokens (the oracle on the GPU's own
    inputs): max |gpu - oracle| / max |oracle| per side, per-layer flag agreement, the oracle's and
    the GPU's normalised error against the exact target (KVCMAS App. A.1 / Fig. 3: ||C_hat - C|| /
    ||C||) and that of the uncorrected re-aligned source, on matched layers."""
    sp = data.spec
    fr = O.inv_freq(sp.head_dim, sp.theta)
    err = {"k": 0.0, "v": 0.0}
    agree, n_flag = 0, 0
    m02, m02_oracle, m02_none = [], [], []
    t0 = time.perf_counter()
    for i, l in enumerate(layers):
        ref = O.correct_layer(data, i)
        for side in ("k", "v"):
            want = O.round_to(ref[f"{side}_out"], sp.dtype)
            got = gpu[f"{side}_out"][i]
            err[side] = max(err[side], float(np.max(np.abs(got - want)) / np.max(np.abs(want))))
        if sp.mode == W.SCORE_PAGES:
            _, _, f = O.gate_decide_pages(np.asarray(ref["q"]), sp.tau, sp.temp_gate, sp.cap(), sp.n_anchors)
        else:
            _, _, f = O.gate_decide_cos(*[np.asarray(x) for x in ref["cos_sums"]], sp.tau, sp.cap(), sp.n_anchors)
        agree += int(f == int(gpu["flags"][1 + l]))
        n_flag += 1
        unrelated = sp.unrelated_layers is not None and gpu["orig_layer"][i] in sp.unrelated_layers
        if not exact or unrelated:
            continue
        for side in ("k", "v"):
            A, B = O.layer_factors(data, i, side, "delta", [0])
            corr = A[0] @ B[0] + W.target_noise(sp, gpu["orig_layer"][i], 0 if side == "k" else 1)
            src = O._np(getattr(data, f"{side}_src")[i])
            if side == "k":
                aligned = O.rope(src, sp.shift, sp.head_dim, fr)
                target = aligned + O.rope(corr, sp.p_tgt, sp.head_dim, fr)
            else:
                aligned = src
                target = src + corr
            m02.append(O.normalized_error(gpu[f"{side}_out"][i], target))
            m02_oracle.append(O.normalized_error(ref[f"{side}_out"], target))
            m02_none.append(O.normalized_error(aligned, target))
    out = {"layers": [int(gpu["orig_layer"][i]) for i in range(len(layers))],
           "max_abs_err_over_max_x": {"k": round(err["k"], 6), "v": round(err["v"], 6), "bound": 2.0 ** -7},
           "layer_flags_agree": f"{agree}/{n_flag}",
           "oracle_s": round(time.perf_counter() - t0, 2)}
    if m02:
        out["normalised_error_vs_exact_target"] = {"gpu": round(float(np.mean(m02)), 5),
                                                   "oracle": round(float(np.mean(m02_oracle)), 5),
                                                   "uncorrected": round(float(np.mean(m02_none)), 5)}
    return out


def cpu_baseline(O, data, n_layers, layers):
    """The fp64 oracle (as it stands) on `layers` of the same hop, all tokens, keys and values;
    tokens/s scaled to all layers."""
    info = host_info()
    S = data.spec.seq_len
    t0 = time.perf_counter()
    for i in range(len(layers)):
        O.correct_layer(data, i)
    dt = time.perf_counter() - t0
    return {"value": round(S / (dt * n_layers / len(layers)), 2), "unit": "tokens/s", "cores": info["blas_threads"],
            "kind": "oracle", "host": info,
            "sample": f"layers {layers} of {n_layers}: {S} tokens x (K, V), scores + weights + gate sums + delta "
                      f"in fp64; {dt:.1f} s, scaled to all layers"}


def cpu_median(O, data, n_layers, layers, runs=3, threads=None):
    """Median of `runs` oracle runs on `layers` (optionally with the BLAS pool limited)."""
    from contextlib import nullcontext
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(threads) if threads else nullcontext()
    except Exception:
        ctx = nullcontext()
    ts = []
    with ctx:
        for _ in range(runs):
            t0 = time.perf_counter()
            for i in range(len(layers)):
                O.correct_layer(data, i)
            ts.append(time.perf_counter() - t0)
    dt = statistics.median(ts)
    S = data.spec.seq_len
    return {"value": round(S / (dt * n_layers / len(layers)), 2), "unit": "tokens/s",
            "median_s": round(dt, 3), "runs": runs, "layers": layers, "threads": threads or host_info()["blas_threads"]}


def measure_c2(kvc, torch, W, data, steps=10, warmup=2):
    """The 4096-token Llama-3.1-8B-shaped hop (32 layers x 8x128, 20 anchors at rank 32, start
    position and shift from the seeded specification), keys placed at p_src on the device by the
    library's re-alignment.  Returns the timing and the GPU's inputs / outputs of sampled layers
    for the oracle leg."""
    sp = data.spec
    k, v = data.k_src.to("cuda"), data.v_src.to("cuda")
    shp = kvc.shape_of(sp.n_layers, sp.seq_len, sp.n_kv_heads, sp.head_dim)
    kvc.align_rope(k, k, shp, 0, sp.p_src)
    ko, vo = torch.empty_like(k), torch.empty_like(v)
    pool = kvc.pool_from(data, "cuda")
    prm_fn = lambda tr: kvc.params_of(sp.tau, sp.temp_gate, sp.temp_weight, sp.gate_len, sp.mode, 0, tr)
    ws = torch.empty((kvc.correct_hop_workspace(shp, pool, prm_fn(None)),), dtype=torch.uint8, device="cuda")
    ms, _, per_kernel, res = time_hop(kvc, torch, k, v, ko, vo, shp, sp, pool, prm_fn, ws, steps, warmup)
    L, S, D, N, r = sp.n_layers, sp.seq_len, sp.d_model, sp.n_anchors, sp.rank_base
    nbytes = 2 * L * S * D * (2 + 2) + 2 * L * N * (2 * r) * (S + D) * 2
    flops = 8 * L * S * D * N * r
    flags = res.flags.cpu().tolist()
    out = {"workload": f"{L} layers x {S} tokens x {sp.n_kv_heads}x{sp.head_dim} bf16, {N} anchors at rank {r}, "
                       f"p_src {sp.p_src}, shift {sp.shift}",
           "ms": round(ms, 4), "tokens_per_s": round(S / (ms / 1e3), 1), "algorithmic_bytes": nbytes,
           "mfma_flops": flops, "hbm_frac": round(nbytes / (ms / 1e3) / PEAK_HBM, 4),
           "mfma_frac": round(flops / (ms / 1e3) / PEAK_MFMA_BF16, 4),
           "kernels_ms": {n: round(statistics.median(t), 4) for n, t in per_kernel.items()},
           "flags": {"hop": flags[0], "layers_flagged": sum(1 for f in flags[1:] if f)}}
    # the flagged fraction over the per-layer gates (reuse ratio of this hop's layers)
    out["accepted_layer_fraction"] = round(sum(1 for f in flags[1:] if not f) / L, 4)
    res2 = kvc.correct_hop(k, v, ko, vo, shp, sp.p_src, sp.p_tgt, pool, prm_fn(None), workspace=ws,
                           want_weights=True)
    torch.cuda.synchronize()
    layers = [0, 15, 31]
    idx = torch.tensor(layers, device="cuda")
    art = {"layers": layers, "k_src": k.index_select(0, idx).cpu(),
           "gpu": {"k_out": ko.index_select(0, idx).double().cpu().numpy(),
                   "v_out": vo.index_select(0, idx).double().cpu().numpy(),
                   "flags": res2.flags.cpu().numpy(), "orig_layer": layers}}
    del k, v, ko, vo, pool, ws
    torch.cuda.empty_cache()
    return out, art


def measure_c5(kvc, torch, W, data, p=32, q=3, steps=5):
    """KVCMAS Sec. 3.3 Eq. 7 then Eq. 8 at the rank-128 configuration: dense fp32 deltas
    (4096 x 1024 per layer and side, Gaussian factors with i^-1.5 column scales, drawn on the
    device) factorised at rank 128 by the refresh, written as anchor 0's delta factors (bf16) of a
    10-anchor pool, then the rank-128 correction of the 32-layer 4096-token hop.  Timed as one
    pipeline: refresh, the factor copies into the pool, the correction."""
    sp = data.spec
    L, S, D, r = sp.n_layers, sp.seq_len, sp.d_model, sp.rank_delta
    k, v = data.k_src.to("cuda"), data.v_src.to("cuda")
    ko, vo = torch.empty_like(k), torch.empty_like(v)
    pool = kvc.pool_from(data, "cuda")
    shp = kvc.shape_of(L, S, sp.n_kv_heads, sp.head_dim)
    g = torch.Generator(device="cuda").manual_seed(5)
    sc = torch.arange(1, D + 1, device="cuda", dtype=torch.float32) ** -1.5
    z = torch.empty((2 * L, S, D), device="cuda")
    for m in range(2 * L):
        a = torch.randn((S, D), device="cuda", generator=g) * sc[None, :]
        z[m] = a @ (torch.randn((D, D), device="cuda", generator=g) / D ** 0.5)
    ws_svd = torch.empty((kvc.svd_workspace_size(2 * L, S, D, r, p),), dtype=torch.uint8, device="cuda")
    a_out = torch.empty((2 * L, S, r), dtype=torch.bfloat16, device="cuda")
    b_out = torch.empty((2 * L, r, D), dtype=torch.bfloat16, device="cuda")
    prm = kvc.params_of(sp.tau, sp.temp_gate, sp.temp_weight, sp.gate_len, sp.mode, 0, None)
    ws = torch.empty((kvc.correct_hop_workspace(shp, pool, prm),), dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream()

    def pipeline():
        kvc.anchor_refresh_svd(z, r, oversample=p, power_iters=q, workspace=ws_svd, a_out=a_out, b_out=b_out)
        pool.deltaA_k[:, :S].copy_(a_out[0::2])
        pool.deltaB_k[:, 0].copy_(b_out[0::2])
        pool.deltaA_v[:, :S].copy_(a_out[1::2])
        pool.deltaB_v[:, 0].copy_(b_out[1::2])
        kvc.correct_hop(k, v, ko, vo, shp, sp.p_src, sp.p_tgt, pool, prm, workspace=ws)

    pipeline()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for e in evs:
        e[0].record(st)
        kvc.anchor_refresh_svd(z, r, oversample=p, power_iters=q, workspace=ws_svd, a_out=a_out, b_out=b_out)
        e[1].record(st)
        pool.deltaA_k[:, :S].copy_(a_out[0::2])
        pool.deltaB_k[:, 0].copy_(b_out[0::2])
        pool.deltaA_v[:, :S].copy_(a_out[1::2])
        pool.deltaB_v[:, 0].copy_(b_out[1::2])
        e[2].record(st)
        kvc.correct_hop(k, v, ko, vo, shp, sp.p_src, sp.p_tgt, pool, prm, workspace=ws)
        e[3].record(st)
    torch.cuda.synchronize()
    med = lambda i, j: statistics.median(e[i].elapsed_time(e[j]) for e in evs)
    t_svd, t_copy, t_cor, t_all = med(0, 1), med(1, 2), med(2, 3), med(0, 3)
    del z, ws_svd, a_out, b_out, k, v, ko, vo, pool, ws
    torch.cuda.empty_cache()
    return {"workload": f"refresh of {2 * L} fp32 deltas {S}x{D} at rank {r} (oversample {p}, {q} power "
                        f"iterations) into anchor 0, then the rank-{r} correction with {sp.n_anchors} anchors "
                        f"({L} layers x {S} tokens x {sp.n_kv_heads}x{sp.head_dim} bf16)",
            "ms": round(t_all, 3), "refresh_ms": round(t_svd, 3), "factor_copy_ms": round(t_copy, 3),
            "correction_ms": round(t_cor, 3), "tokens_per_s_correction": round(S / (t_cor / 1e3), 1)}


def time_hop(kvc, torch, k, v, ko, vo, shp, sp, pool, prm_fn, ws, steps, warmup, trace=True):
    for _ in range(warmup):
        kvc.correct_hop(k, v, ko, vo, shp, sp.p_src, sp.p_tgt, pool, prm_fn(None), workspace=ws)
    torch.cuda.synchronize()
    traces = [kvc.KernelTrace(16) for _ in range(steps)] if trace else [None] * steps
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    t0 = time.perf_counter()
    for i in range(steps):
        res = kvc.correct_hop(k, v, ko, vo, shp, sp.p_src, sp.p_tgt, pool, prm_fn(traces[i]), workspace=ws)
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    per_kernel = {}
    for tr in traces:
        if tr is None:
            continue
        for name, t in tr.results():
            per_kernel.setdefault(name, []).append(t)
        tr.close()
    return ms, wall, per_kernel, res


def measure_protocol(kvc, torch, k, v, ko, vo, shp, sp, pool, prm, reps=20, warmup=5):
    """One hop timed repetition by repetition: `warmup` untimed calls, then `reps` calls each
    bracketed by its own events, with the 256 MB Infinity Cache flushed in between by a 512 MiB
    fill outside the bracket; median, p10 and p90 for the fused call (kvc_correct_hop) and for
    the unfused sequence (kvc_match_anchors, which writes the token weights to memory, then
    kvc_apply_lowrank_delta; the re-alignment is fused into both), and the standalone key
    re-alignment (kvc_align_rope) as an HBM stream."""
    import numpy as np
    dev = k.device
    st = torch.cuda.current_stream()
    L, S, D = shp.n_layers, shp.seq_len, shp.n_kv_heads * shp.head_dim
    N = len(pool.anchor_len)
    flush = torch.empty((512 << 20,), dtype=torch.uint8, device=dev)
    m = kvc.alloc_match(L, S, N, dev, want_weights=True)
    ws_c = torch.empty((max(kvc.correct_hop_workspace(shp, pool, prm), 1),), dtype=torch.uint8, device=dev)
    ws_m = torch.empty((max(kvc.workspace_size(kvc.CALL_MATCH, shp, pool, prm), 1),), dtype=torch.uint8, device=dev)
    ws_a = torch.empty((max(kvc.workspace_size(kvc.CALL_APPLY, shp, pool), 1),), dtype=torch.uint8, device=dev)

    def fused():
        kvc.correct_hop(k, v, ko, vo, shp, sp.p_src, sp.p_tgt, pool, prm, workspace=ws_c)

    def unfused():
        kvc.match_anchors(k, v, shp, sp.p_src, pool, prm, out=m, workspace=ws_m)
        kvc.apply_lowrank_delta(k, v, ko, vo, shp, sp.p_src, sp.p_tgt, pool, m.w_k, m.w_v, m.s_cov, workspace=ws_a)

    def align():
        kvc.align_rope(k, ko, shp, sp.p_src, sp.p_tgt)

    def reps_of(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        evs = []
        for i in range(reps):
            flush.fill_(i & 0xff)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            fn()
            e1.record(st)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ts = np.array([a.elapsed_time(b) for a, b in evs])
        return {"median_ms": round(float(np.median(ts)), 4), "p10_ms": round(float(np.percentile(ts, 10)), 4),
                "p90_ms": round(float(np.percentile(ts, 90)), 4)}

    out = {"reps": reps, "warmup": warmup, "flush_bytes": flush.numel(), "fused": reps_of(fused),
           "match_then_apply": reps_of(unfused)}
    al = reps_of(align)
    al["bytes"] = 2 * L * S * D * k.element_size()
    al["achieved_GBps"] = round(al["bytes"] / (al["median_ms"] / 1e3) / 1e9, 1)
    out["align_rope_keys"] = al
    out["fused_tokens_per_s"] = round(S / (out["fused"]["median_ms"] / 1e3), 1)
    out["unfused_over_fused"] = round(out["match_then_apply"]["median_ms"] / out["fused"]["median_ms"], 3)
    del flush, ws_c, ws_m, ws_a, m
    return out


SECTIONS = ("peaks", "hop", "protocol", "second", "c2", "refresh", "chain", "pf", "r128", "c5", "study", "pool", "cpu")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=32, help="smaller values are for quick local runs only")
    ap.add_argument("--seq-len", type=int, default=32768, help="smaller values are for quick local runs only")
    ap.add_argument("--mode", choices=["pages", "cos"], default="pages")
    ap.add_argument("--p-src", type=int, default=512, help="start position of the segment in the source agent")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-second-mode", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the refresh, chained-batch and other sections")
    ap.add_argument("--only", default="", help="comma-separated sections to run (profiling): " + ",".join(SECTIONS))
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the per-hop correction runs on one GPU only; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    want = set(args.only.split(",")) if args.only else set(SECTIONS)
    bad = want - set(SECTIONS)
    if bad:
        print(f"bench.py: unknown sections {sorted(bad)}", file=sys.stderr)
        sys.exit(2)
    if args.no_extra:
        want -= {"refresh", "chain", "pf", "r128", "c5", "study", "pool", "c2"}
    if args.no_second_mode:
        want.discard("second")
    if args.no_cpu_baseline:
        want.discard("cpu")

    import numpy as np  # noqa: F401
    import torch

    from rank_kv_cache_layer_amd import kvc
    from rank_kv_cache_layer_amd import workload as W

    # host-side inputs first: the seeded generator forks worker processes only before the GPU is
    # initialised in this process
    mode = W.SCORE_PAGES if args.mode == "pages" else W.SCORE_COS_R
    sp = W.llama8b_long(n_layers=args.layers, seq_len=args.seq_len, mode=mode)
    data = data_c2 = data_c5 = None
    need_hop = bool(want & {"hop", "protocol", "second", "cpu"})
    if need_hop:
        t0 = time.perf_counter()
        data = W.make_hop(sp)
        log(f"[bench] generated {sp.name}: L={sp.n_layers} S={sp.seq_len} D={sp.d_model} N={sp.n_anchors} "
            f"r={sp.rank_base} in {time.perf_counter() - t0:.1f} s")
    if "c2" in want:
        sp2 = W.llama8b_hop()
        data_c2 = W.make_hop(dataclasses.replace(sp2, p_src=0, p_tgt=sp2.shift))
        data_c2 = dataclasses.replace(data_c2, spec=sp2)   # keys placed at p_src on the device
        log(f"[bench] generated {sp2.name}")
    if want & {"c5", "r128"}:
        data_c5 = W.make_hop(W.llama8b_rank128())
        log("[bench] generated llama8b_r128")

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    kvc.lib()
    dev = "cuda:0"
    out = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"llama8b_hop_{sp.seq_len}tok" if sp.seq_len != 32768 or sp.n_layers != 32
                      else "llama8b_32k_hop", "n_layers": sp.n_layers, "seq_len": sp.seq_len,
                      "n_kv_heads": sp.n_kv_heads, "head_dim": sp.head_dim, "n_anchors": sp.n_anchors,
                      "rank": sp.rank_base, "shift": sp.shift, "score_mode": args.mode,
                      "unrelated_layers": len(sp.unrelated_layers or []), "parallelism": "single-gpu"},
           "roofline": None, "cpu_baseline": None}

    def guarded(key, fn):
        # a failing secondary measurement is recorded and must not hide the headline line
        try:
            return fn()
        except Exception as e:
            log(f"[bench] {key} failed: {type(e).__name__}: {e}")
            out.setdefault("errors", {})[key] = f"{type(e).__name__}: {e}"
            return None

    if "peaks" in want:
        out["measured_peaks"] = guarded("peaks", lambda: measure_peaks(kvc, torch))
        log(f"[bench] measured ceilings: {out['measured_peaks']}")

    art3 = None
    if need_hop:
        k = data.k_src.to(dev)
        v = data.v_src.to(dev)
        ko, vo = torch.empty_like(k), torch.empty_like(v)
        pool = kvc.pool_from(data, dev)
        shp = kvc.shape_of(sp.n_layers, sp.seq_len, sp.n_kv_heads, sp.head_dim)
        # keys are drawn in the canonical frame; place the segment at start position 512 (target
        # 812) with the library's own re-alignment, in place
        kvc.align_rope(k, k, shp, 0, args.p_src)
        sp = dataclasses.replace(sp, p_src=args.p_src, p_tgt=args.p_src + sp.shift)

        def prm_fn(mode_):
            return lambda tr: kvc.params_of(sp.tau, sp.temp_gate, sp.temp_weight, sp.gate_len, mode_, 0, tr)

        ws_bytes = max(kvc.correct_hop_workspace(shp, pool, prm_fn(m)(None)) for m in (W.SCORE_PAGES, W.SCORE_COS_R))
        ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        log(f"[bench] inputs resident on {torch.cuda.get_device_name(0)}; workspace {ws_bytes / 2**20:.0f} MiB")
        S, L, D, N, r = sp.seq_len, sp.n_layers, sp.d_model, sp.n_anchors, sp.rank_base
        if "hop" in want or "cpu" in want:
            ms, wall, per_kernel, res = time_hop(kvc, torch, k, v, ko, vo, shp, sp, pool, prm_fn(mode), ws,
                                                 args.steps, args.warmup)
            flags = res.flags.cpu().tolist()
            log(f"[bench] {args.mode}: {ms:.3f} ms/hop (wall {wall / args.steps * 1e3:.3f} ms), flags hop={flags[0]} "
                f"layers={sum(1 for f in flags[1:] if f)} flagged")
            kernels = {}
            for name, ts in per_kernel.items():
                med = statistics.median(ts)
                kernels[name] = roofline(name, med, kernel_work(name, L, S, D, N, r, r, args.mode),
                                         measured_traffic(name))
            dominant = max(kernels.values(), key=lambda x: x["ms"]) if kernels else None
            hop_bytes = 2 * L * S * D * (2 + 2) + 2 * L * N * (2 * r) * (S + D) * 2
            hop_flops = 8 * L * S * D * N * r
            out.update({"value": round(S / (ms / 1e3), 1), "ms_per_step": round(ms, 4), "roofline": dominant,
                        "kernels": kernels,
                        "hop": {"ms": round(ms, 4), "algorithmic_bytes": hop_bytes, "mfma_flops": hop_flops,
                                "hbm_frac": round(hop_bytes / (ms / 1e3) / PEAK_HBM, 4),
                                "mfma_frac": round(hop_flops / (ms / 1e3) / PEAK_MFMA_BF16, 4)},
                        "flags": {"hop": flags[0], "layers_flagged": sum(1 for f in flags[1:] if f),
                                  "accepted_layer_fraction": round(sum(1 for f in flags[1:] if not f) / L, 4)}})
            if "cpu" in want:
                # the GPU's inputs and outputs of sampled layers, for the oracle leg
                lay = [0, 1, 2]
                idx = torch.tensor(lay, device=dev)
                art3 = {"layers": lay, "k_src": k.index_select(0, idx).cpu(),
                        "gpu": {"k_out": ko.index_select(0, idx).double().cpu().numpy(),
                                "v_out": vo.index_select(0, idx).double().cpu().numpy(),
                                "flags": res.flags.cpu().numpy(), "orig_layer": lay}}
        if "protocol" in want:
            out["protocol"] = guarded("protocol", lambda: measure_protocol(kvc, torch, k, v, ko, vo, shp, sp, pool,
                                                                           prm_fn(mode)(None)))
            log(f"[bench] per-repetition protocol (cache flushed): {out['protocol']}")
        if "second" in want:
            def second():
                m2 = W.SCORE_COS_R if mode == W.SCORE_PAGES else W.SCORE_PAGES
                ms2, _, pk2, _ = time_hop(kvc, torch, k, v, ko, vo, shp, sp, pool, prm_fn(m2), ws,
                                          max(3, args.steps // 4), 1)
                return {"mode": "cos_r" if m2 == W.SCORE_COS_R else "pages", "ms_per_hop": round(ms2, 4),
                        "tokens_per_s": round(S / (ms2 / 1e3), 1),
                        "kernels_ms": {n: round(statistics.median(t), 4) for n, t in pk2.items()}}
            out["second_mode"] = guarded("second", second)
            log(f"[bench] second mode: {out['second_mode']}")
        del k, v, ko, vo, pool, ws
        torch.cuda.empty_cache()

    art2 = None
    if "c2" in want:
        log("[bench] 4096-token hop (32 layers, 20 anchors at rank 32) ...")
        r2 = guarded("c2", lambda: measure_c2(kvc, torch, W, data_c2))
        if r2 is not None:
            out["c2_hop"], art2 = r2
        log(f"[bench] c2: {out.get('c2_hop')}")
    for key, want_key, msg, fn in (
            ("refresh", "refresh", "anchor refresh (64 x 4096 x 1024, rank 128)",
             lambda: measure_refresh(kvc, torch, oracle="cpu" in want)),
            ("chained_batch", "chain", "chained batch (8 requests x 3 hops, 8192 tokens)",
             lambda: measure_chain(kvc, torch, W)),
            ("pf_delta", "pf", "preconstructed rank-8 correction, weight 1 (32 layers x 32768 tokens)",
             lambda: measure_pf_delta(kvc, torch)),
            ("rank128_hop", "r128", "rank-128 correction (32 layers x 4096 tokens, 10 anchors)",
             lambda: measure_rank128(kvc, torch, W, data_c5)),
            ("c5_pipeline", "c5", "refresh into anchor 0, then the rank-128 correction",
             lambda: measure_c5(kvc, torch, W, data_c5)),
            ("chain_study", "study", "chained vs non-chained correction error along A0 -> A3 (8 layers x 4096 x 1024)",
             lambda: measure_study(torch)),
            ("pool_insert", "pool", "pool update after a fallback (32 layers x 4096 tokens, rank 32)",
             lambda: measure_pool_insert(kvc, torch, oracle="cpu" in want))):
        if want_key in want:
            log(f"[bench] {msg} ...")
            out[key] = guarded(want_key, fn)
            log(f"[bench] {want_key}: {out[key]}")

    if "cpu" in want and art3 is not None:
        guarded("cpu", lambda: cpu_section(O_loader(), out, data, data_c2, art2, art3, sp, dev, kvc, torch, W))

    print(json.dumps(out), flush=True)


def O_loader():
    from oracle import kvc_oracle as O
    return O


def cpu_section(O, out, data, data_c2, art2, art3, sp, dev, kvc, torch, W):
    """The oracle's baselines (bounded samples of the 32768-, 4096-token and tiny hops) and the quality of the GPU's
    outputs of sampled layers against the oracle and the exact target."""
    log("[bench] timing the fp64 oracle on bounded samples, and parity / quality on sampled layers ...")
    d3 = _layers_of(data, art3["layers"], k_src=art3["k_src"])
    d3 = dataclasses.replace(d3, spec=dataclasses.replace(d3.spec, p_src=sp.p_src, p_tgt=sp.p_tgt,
                                                          n_layers=len(art3["layers"]),
                                                          unrelated_layers=sp.unrelated_layers))
    out["cpu_baseline"] = cpu_baseline(O, d3, sp.n_layers, art3["layers"])
    log(f"[bench] oracle: {out['cpu_baseline']['value']} tokens/s ({out['cpu_baseline']['sample']})")
    base = {"c3": dict(out["cpu_baseline"])}
    quality = {"c3": hop_quality(O, W, d3, art3["gpu"], art3["layers"])}
    if art2 is not None:
        sp2 = data_c2.spec
        d2 = _layers_of(data_c2, art2["layers"], k_src=art2["k_src"])
        base["c2"] = cpu_median(O, d2, sp2.n_layers, art2["layers"])
        quality["c2"] = hop_quality(O, W, d2, art2["gpu"], art2["layers"])
        quality["c2"]["accepted_layer_fraction"] = out["c2_hop"]["accepted_layer_fraction"]
    # the tiny fp32 workload: whole hop, median of 3, also on one thread; GPU parity beside it
    dt1 = W.make_hop(W.tiny(), place_keys=lambda x, p_: O.rope(x, p_, 64))
    sp1 = dt1.spec
    base["c1"] = cpu_median(O, dt1, sp1.n_layers, list(range(sp1.n_layers)))
    base["c1_single_thread"] = cpu_median(O, dt1, sp1.n_layers, list(range(sp1.n_layers)), threads=1)
    k1, v1 = dt1.k_src.to(dev), dt1.v_src.to(dev)
    ko1, vo1 = torch.empty_like(k1), torch.empty_like(v1)
    shp1 = kvc.shape_of(sp1.n_layers, sp1.seq_len, sp1.n_kv_heads, sp1.head_dim)
    res1 = kvc.correct_hop(k1, v1, ko1, vo1, shp1, sp1.p_src, sp1.p_tgt, kvc.pool_from(dt1, dev),
                           kvc.params_of(sp1.tau, sp1.temp_gate, sp1.temp_weight, sp1.gate_len, sp1.mode))
    torch.cuda.synchronize()
    ref1 = O.correct_hop(dt1)
    quality["c1"] = {"max_abs_err_over_max_x": {
        s_: round(float(np.max(np.abs(t.double().cpu().numpy() - ref1[f"{s_}_out"])) /
                        np.max(np.abs(ref1[f"{s_}_out"]))), 9) for s_, t in (("k", ko1), ("v", vo1))},
        "bound": 1e-5, "flags_equal": bool(np.array_equal(res1.flags.cpu().numpy(), ref1["flags"]))}
    out["cpu_baselines"] = base
    out["quality"] = quality
    log(f"[bench] oracle baselines: {base}")
    log(f"[bench] quality: {quality}")


if __name__ == "__main__":
    main()
