#!/usr/bin/env python3
"""Throughput of the MiMo-V2-Flash hybrid attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic inputs:
  1. SWA prefill layer: 4 sequences x 8192 tokens, window 129, sink;
  2. GA prefill layer: 1 sequence x 32768 tokens, sink;
  3. one decode step for 128 sequences with contexts uniform in [4096, 262144]:
     SWA layer (128-slot ring) and GA layer (full bf16 pool, split-K), each
     attend-then-append, then the host-visible context counters advance.
Shapes: 64 query heads over 4 KV heads, head dims 192 (q/k) and 128 (v); all
inputs N(0,1) bf16 and sinks N(0,1) fp32, seeded; everything resident in HBM
before timing starts.

Prints ONE JSON line.  `value` is the step's algorithmic attention FLOPs
(640 per unmasked query-key-head triple, prefill and decode) divided by the
step time; per-phase TFLOP/s, tokens/s and GB/s are in `breakdown`.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from global_attention_mimo_amd import binding as B  # noqa: E402
from global_attention_mimo_amd import prof  # noqa: E402
from global_attention_mimo_amd import synth  # noqa: E402

HQ, HKV, DQK, DV, W = 64, 4, 192, 128, 129
FLOP_PER_TRIPLE = 2 * (DQK + DV)                      # 640
TOKEN_BYTES = HQ * DQK * 2 + HKV * (DQK + DV) * 2 + HQ * DV * 2 + HQ * 4  # q,k,v,o,lse = 43,776
KV_TOKEN_BYTES = HKV * (DQK + DV) * 2                 # 2,560
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0
METRIC = "attention TFLOP/s (prefill) + decode tokens/s & HBM GB/s, SWA and GA, 1 GPU"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prefill_pairs(lengths, layer_type, window=W):
    tot = 0
    for L in lengths:
        if layer_type == 1:
            tot += L * (L + 1) // 2
        else:
            n = min(L, window)
            tot += n * (n + 1) // 2 + (L - n) * window
    return tot


def decode_stats(ctx, layer_type, window=W):
    ctx = np.asarray(ctx, dtype=np.int64)
    if layer_type == 1:
        keys = ctx + 1
        cached = ctx
    else:
        keys = np.minimum(ctx + 1, window)
        cached = np.minimum(ctx, window - 1)
    flops = int(keys.sum()) * HQ * FLOP_PER_TRIPLE
    bytes_ = int(cached.sum()) * KV_TOKEN_BYTES + len(ctx) * TOKEN_BYTES
    return flops, bytes_


def measured_traffic(record="profiles/prefill_ga_1x32768_traffic.json"):
    """HBM bytes per GA-prefill launch from the rocprofv3 FETCH_SIZE/WRITE_SIZE record
    that `python -m global_attention_mimo_amd.prof report --suite step` writes
    (copy-calibrated), or None when the kernel code changed since it was taken."""
    path = os.path.join(ROOT, record)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if prof.code_digest(rec["sources"]) != rec.get("code_sha256"):
        return None
    return rec["read_bytes"] + rec["write_bytes"]


def chunk_rows(dims, ga, swa, reps=5):
    """Chunked prefill (prefill continuing cached sequences), timed apart from the
    step: GA, one sequence with its first 28672 positions cached and the last
    4096 as the chunk (the GA prefill input, split); SWA, the 4 x 8192 input as
    chunks that continue 8192 cached positions each (the ring holds the last 128).
    Caches are filled by the library's append before timing."""
    dev = "cuda"
    res = {}
    # GA: pool rows 0..32767 for the sequence, first 28672 appended.
    c, n = 28672, 4096
    kc = torch.zeros((32768, HKV, DQK), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros((32768, HKV, DV), dtype=torch.bfloat16, device=dev)
    base = torch.zeros(1, dtype=torch.int64, device=dev)
    cap = torch.full((1,), 32768, dtype=torch.int64, device=dev)
    zero = torch.zeros(1, dtype=torch.int32, device=dev)
    B.mimo_kv_append(dims, 1, ga.k[:c], ga.v[:c], torch.tensor([0, c], dtype=torch.int32, device=dev), zero, 1, c,
                     kc, vc, base, cap)
    cu = torch.tensor([0, n], dtype=torch.int32, device=dev)
    ctx = torch.full((1,), c, dtype=torch.int32, device=dev)
    q, k, v = ga.q[c:].contiguous(), ga.k[c:].contiguous(), ga.v[c:].contiguous()
    out = torch.empty((n, HQ, DV), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((n, HQ), dtype=torch.float32, device=dev)
    call = lambda: B.mimo_attn_prefill_chunk(dims, 1, q, k, v, cu, 1, n, kc, vc, base, ctx, ga.sink, out, lse)
    ms = _time_ms(call, reps)
    pairs = n * c + n * (n + 1) // 2
    tfs = pairs * HQ * FLOP_PER_TRIPLE / (ms * 1e-3) / 1e12
    res["prefill_chunk_ga"] = {"workload": "1 sequence, 28672 cached + 4096 new", "ms": ms, "TFLOP/s": tfs,
                               "frac_mfma_peak": tfs / PEAK_BF16_TFLOPS}
    del kc, vc, q, k, v, out, lse
    # SWA: ring [4][128] after appending 8192 positions per sequence; chunks are the 4 x 8192 input.
    kc = torch.zeros((4, W - 1, HKV, DQK), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros((4, W - 1, HKV, DV), dtype=torch.bfloat16, device=dev)
    zeros = torch.zeros(4, dtype=torch.int32, device=dev)
    B.mimo_kv_append(dims, 0, swa.k, swa.v, swa.cu_seqlens, zeros, 4, swa.k.shape[0], kc, vc, None, None)
    ctx = torch.full((4,), 8192, dtype=torch.int32, device=dev)
    out = torch.empty((swa.q.shape[0], HQ, DV), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((swa.q.shape[0], HQ), dtype=torch.float32, device=dev)
    call = lambda: B.mimo_attn_prefill_chunk(dims, 0, swa.q, swa.k, swa.v, swa.cu_seqlens, 4, 8192, kc, vc, None,
                                             ctx, swa.sink, out, lse)
    ms = _time_ms(call, reps)
    nbytes = swa.q.shape[0] * TOKEN_BYTES + 4 * (W - 1) * KV_TOKEN_BYTES
    res["prefill_chunk_swa"] = {"workload": "4 sequences, 8192 cached + 8192 new each", "ms": ms,
                                "TFLOP/s": 4 * 8192 * W * HQ * FLOP_PER_TRIPLE / (ms * 1e-3) / 1e12,
                                "GB/s": nbytes / (ms * 1e-3) / 1e9,
                                "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    return res


def paged_rows(dims, dga, ctx, max_ctx, ws, ga, page_size=16, reps=5):
    """Paged GA pool, timed apart from the step: the decode step's GA attention
    (128 sequences at the contexts the timed steps left) with the pool in pages
    of 16 rows on a seeded random page order, next to the same call over the
    contiguous pool; and the GA chunk (28672 cached + 4096 new) over a paged pool."""
    dev = "cuda"
    res = {}
    ctx_list = [int(c) for c in ctx.cpu()]
    table, npages = synth.paged_block_table(ctx_list, page_size, seed=1, device=dev)
    kp = torch.empty((npages * page_size, HKV, DQK), dtype=torch.bfloat16, device=dev)
    vp = torch.empty((npages * page_size, HKV, DV), dtype=torch.bfloat16, device=dev)
    for b, c in enumerate(ctx_list):
        j = torch.arange(c, device=dev)
        dst = table[b, j // page_size].long() * page_size + j % page_size
        src = int(dga.kv_base[b]) + j
        kp[dst] = dga.k_cache[src]
        vp[dst] = dga.v_cache[src]
    pages = B.make_pages(table, page_size, npages)
    Bd = len(ctx_list)
    out = torch.empty((Bd, HQ, DV), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Bd, HQ), dtype=torch.float32, device=dev)
    paged = lambda: B.mimo_attn_decode_paged(dims, dga.q, dga.k_new, dga.v_new, kp, vp, pages, ctx, Bd, max_ctx, 0,
                                             dga.sink, out, lse, ws)
    flat = lambda: B.mimo_attn_decode(dims, 1, dga.q, dga.k_new, dga.v_new, dga.k_cache, dga.v_cache, dga.kv_base,
                                      ctx, Bd, max_ctx, 0, dga.sink, out, lse, ws)
    ms_p, ms_f = _time_ms(paged, reps), _time_ms(flat, reps)
    _, nbytes = decode_stats(ctx_list, 1)
    res["decode_ga_paged"] = {"workload": f"decode step B=128, GA pool in pages of {page_size} (random order)",
                              "ms": ms_p, "tokens/s": Bd / (ms_p * 1e-3), "GB/s": nbytes / (ms_p * 1e-3) / 1e9,
                              "frac_hbm_peak": nbytes / (ms_p * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                              "contiguous_ms": ms_f}
    del kp, vp, table
    torch.cuda.empty_cache()
    # GA chunk over a paged pool: 28672 cached positions in pages of 16.
    c, n = 28672, 4096
    table, npages = synth.paged_block_table([c], page_size, seed=2, extra_tokens=0, device=dev)
    kp = torch.empty((npages * page_size, HKV, DQK), dtype=torch.bfloat16, device=dev)
    vp = torch.empty((npages * page_size, HKV, DV), dtype=torch.bfloat16, device=dev)
    zero = torch.zeros(1, dtype=torch.int32, device=dev)
    B.kv_append_paged(ga.k[:c].contiguous(), ga.v[:c].contiguous(), torch.tensor([0, c], dtype=torch.int32,
                      device=dev), zero, kp, vp, table, page_size, dims=dims)
    pages = B.make_pages(table, page_size, npages)
    cu = torch.tensor([0, n], dtype=torch.int32, device=dev)
    ctxc = torch.full((1,), c, dtype=torch.int32, device=dev)
    q, k, v = ga.q[c:].contiguous(), ga.k[c:].contiguous(), ga.v[c:].contiguous()
    out = torch.empty((n, HQ, DV), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((n, HQ), dtype=torch.float32, device=dev)
    call = lambda: B.mimo_attn_prefill_chunk_paged(dims, q, k, v, cu, 1, n, kp, vp, pages, ctxc, ga.sink, out, lse)
    ms = _time_ms(call, reps)
    tfs = (n * c + n * (n + 1) // 2) * HQ * FLOP_PER_TRIPLE / (ms * 1e-3) / 1e12
    res["prefill_chunk_ga_paged"] = {"workload": f"1 sequence, 28672 cached (pages of {page_size}) + 4096 new",
                                     "ms": ms, "TFLOP/s": tfs, "frac_mfma_peak": tfs / PEAK_BF16_TFLOPS}
    del kp, vp, q, k, v, out, lse
    torch.cuda.empty_cache()
    return res


def fp8_rows(dims, dga, ctx, max_ctx, ws, ga, page_size=16, reps=5):
    """FP8 (OCP E4M3) GA pool, timed apart from the step: the decode step's GA
    attention (128 sequences at the contexts the timed steps left) over the
    pool quantised by the library's append with one scale per KV head (an amax
    calibration of N(0,1) data: 4.5 / 448), next to the same call over the bf16
    pool, and over the same codes in pages of 16 (random order).  The
    quantising append of all cached positions is timed too, and the GA chunk
    (28672 cached + 4096 new) over an FP8 pool next to the bf16 one."""
    dev = "cuda"
    ctx_list = [int(c) for c in ctx.cpu()]
    Bd = len(ctx_list)
    rows = dga.k_cache.shape[0]
    k8 = torch.empty((rows, HKV, DQK), dtype=torch.uint8, device=dev)
    v8 = torch.empty((rows, HKV, DV), dtype=torch.uint8, device=dev)
    ks = torch.full((HKV,), 4.5 / 448, dtype=torch.float32, device=dev)
    vs = torch.full((HKV,), 4.5 / 448, dtype=torch.float32, device=dev)
    # every cached row of the pool, as one packed append per sequence region
    cu = torch.tensor(np.concatenate([[0], np.cumsum(dga.kv_capacity.cpu().numpy())]), dtype=torch.int32, device=dev)
    zeros = torch.zeros(Bd, dtype=torch.int32, device=dev)
    app = lambda: B.mimo_kv_append_fp8(dims, dga.k_cache, dga.v_cache, cu, zeros, Bd, rows, k8, v8, dga.kv_base,
                                       dga.kv_capacity, ks, vs)
    ms_app = _time_ms(app, 2)
    out = torch.empty((Bd, HQ, DV), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Bd, HQ), dtype=torch.float32, device=dev)
    f8 = lambda: B.mimo_attn_decode_fp8(dims, dga.q, dga.k_new, dga.v_new, k8, v8, dga.kv_base, ks, vs, ctx, Bd,
                                        max_ctx, 0, dga.sink, out, lse, ws)
    bf = lambda: B.mimo_attn_decode(dims, 1, dga.q, dga.k_new, dga.v_new, dga.k_cache, dga.v_cache, dga.kv_base,
                                    ctx, Bd, max_ctx, 0, dga.sink, out, lse, ws)
    ms_8, ms_b = _time_ms(f8, reps), _time_ms(bf, reps)
    cached = int(sum(ctx_list))
    nbytes = cached * KV_TOKEN_BYTES // 2 + Bd * TOKEN_BYTES
    res = {"decode_ga_fp8": {"workload": "decode step B=128, GA pool of E4M3 codes (1280 B per cached token)",
                             "ms": ms_8, "tokens/s": Bd / (ms_8 * 1e-3), "GB/s": nbytes / (ms_8 * 1e-3) / 1e9,
                             "frac_hbm_peak": nbytes / (ms_8 * 1e-3) / 1e9 / PEAK_HBM_GBPS, "bf16_pool_ms": ms_b,
                             "speedup_vs_bf16_pool": ms_b / ms_8},
           "append_fp8_bulk": {"workload": f"quantise {rows} pool rows (bf16 -> E4M3)", "ms": ms_app,
                               "GB/s": rows * (KV_TOKEN_BYTES + KV_TOKEN_BYTES // 2) / (ms_app * 1e-3) / 1e9}}
    # the same codes in pages of 16 rows, random page order
    table, npages = synth.paged_block_table(ctx_list, page_size, seed=1, device=dev)
    kp = torch.empty((npages * page_size, HKV, DQK), dtype=torch.uint8, device=dev)
    vp = torch.empty((npages * page_size, HKV, DV), dtype=torch.uint8, device=dev)
    for b, c in enumerate(ctx_list):
        j = torch.arange(c, device=dev)
        dst = table[b, j // page_size].long() * page_size + j % page_size
        src = int(dga.kv_base[b]) + j
        kp[dst] = k8[src]
        vp[dst] = v8[src]
    del k8, v8
    pages = B.make_pages(table, page_size, npages)
    p8 = lambda: B.mimo_attn_decode_fp8_paged(dims, dga.q, dga.k_new, dga.v_new, kp, vp, pages, ks, vs, ctx, Bd,
                                              max_ctx, 0, dga.sink, out, lse, ws)
    ms_p = _time_ms(p8, reps)
    res["decode_ga_fp8_paged"] = {"workload": f"decode step B=128, E4M3 pool in pages of {page_size} (random order)",
                                  "ms": ms_p, "tokens/s": Bd / (ms_p * 1e-3), "GB/s": nbytes / (ms_p * 1e-3) / 1e9,
                                  "frac_hbm_peak": nbytes / (ms_p * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                                  "contiguous_fp8_ms": ms_8}
    del kp, vp, table
    torch.cuda.empty_cache()
    # GA chunk over an FP8 pool: 28672 cached positions quantised by the append, then 4096 new tokens.
    c, n = 28672, 4096
    kc8 = torch.zeros((32768, HKV, DQK), dtype=torch.uint8, device=dev)
    vc8 = torch.zeros((32768, HKV, DV), dtype=torch.uint8, device=dev)
    base = torch.zeros(1, dtype=torch.int64, device=dev)
    cap = torch.full((1,), 32768, dtype=torch.int64, device=dev)
    zero = torch.zeros(1, dtype=torch.int32, device=dev)
    B.mimo_kv_append_fp8(dims, ga.k[:c].contiguous(), ga.v[:c].contiguous(),
                         torch.tensor([0, c], dtype=torch.int32, device=dev), zero, 1, c, kc8, vc8, base, cap, ks, vs)
    cu1 = torch.tensor([0, n], dtype=torch.int32, device=dev)
    ctxc = torch.full((1,), c, dtype=torch.int32, device=dev)
    q, k, v = ga.q[c:].contiguous(), ga.k[c:].contiguous(), ga.v[c:].contiguous()
    out_c = torch.empty((n, HQ, DV), dtype=torch.bfloat16, device=dev)
    lse_c = torch.empty((n, HQ), dtype=torch.float32, device=dev)
    call = lambda: B.mimo_attn_prefill_chunk_fp8(dims, q, k, v, cu1, 1, n, kc8, vc8, base, ks, vs, ctxc, ga.sink,
                                                 out_c, lse_c)
    ms = _time_ms(call, reps)
    tfs = (n * c + n * (n + 1) // 2) * HQ * FLOP_PER_TRIPLE / (ms * 1e-3) / 1e12
    res["prefill_chunk_ga_fp8"] = {"workload": "1 sequence, 28672 cached (E4M3 pool) + 4096 new", "ms": ms,
                                   "TFLOP/s": tfs, "frac_mfma_peak": tfs / PEAK_BF16_TFLOPS}
    del kc8, vc8, q, k, v, out_c, lse_c
    torch.cuda.empty_cache()
    return res


def backward_rows(dims, ga, swa, out_ga, lse_ga, out_swa, lse_swa, reps=3):
    """Prefill backward (dq, dk, dv, dsink of sum(dout * out)) on the step's two
    prefill inputs, timed apart from the step; dout is seeded N(0,1) bf16.
    Algorithmic flops: 1664 per unmasked (query, key, head) triple (recomputed
    S 384, dP 256, dV 256, dQ 384, dK 384)."""
    dev = "cuda"
    res = {}
    g = torch.Generator(device=dev).manual_seed(7)
    for name, x, out, lse, lt, L, n in (("backward_ga", ga, out_ga, lse_ga, 1, 32768, 1),
                                         ("backward_swa", swa, out_swa, lse_swa, 0, 8192, 4)):
        T = x.q.shape[0]
        dout = torch.randn((T, HQ, DV), generator=g, device=dev).to(torch.bfloat16)
        dq, dk, dv = torch.empty_like(x.q), torch.empty_like(x.k), torch.empty_like(x.v)
        ds = torch.empty(HQ, dtype=torch.float32, device=dev)
        ws = torch.empty(B.mimo_attn_prefill_backward_workspace_size(dims, T) // 4 + 4, dtype=torch.float32,
                         device=dev)
        call = lambda: B.mimo_attn_prefill_backward(dims, lt, x.q, x.k, x.v, out, lse, dout, x.cu_seqlens, n, L, T,
                                                    x.sink, dq, dk, dv, ds, ws)
        ms = _time_ms(call, reps)
        flops = prefill_pairs([L] * n, lt) * HQ * 1664
        tfs = flops / (ms * 1e-3) / 1e12
        res[name] = {"workload": f"{n} x {L} tokens, {'GA' if lt else 'SWA'}", "ms": ms, "TFLOP/s": tfs,
                     "frac_mfma_peak": tfs / PEAK_BF16_TFLOPS}
        del dout, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return res


def rope_rows(dims, ga, reps=5):
    """Rotary embedding of the GA prefill input's q and k in place (1 x 32768
    tokens, rotary dims 64 of 192, theta 5e6), timed apart from the step; bytes
    are the rotated dims read and written."""
    dev = "cuda"
    q, k = ga.q.clone(), ga.k.clone()
    pos = torch.arange(q.shape[0], dtype=torch.int32, device=dev)
    call = lambda: B.mimo_rope_apply(dims, q, k, pos, q.shape[0], 5e6, 64)
    ms = _time_ms(call, reps)
    nbytes = q.shape[0] * (HQ + HKV) * 64 * 2 * 2
    del q, k
    torch.cuda.empty_cache()
    return {"rope_qk": {"workload": "1 x 32768 tokens, q and k, rotary dims 64, theta 5e6", "ms": ms,
                        "GB/s": nbytes / (ms * 1e-3) / 1e9, "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}}


def swa_decode_rotated_rows(dims, ctx, sets=8, rounds=4):
    """SWA decode of the step's batch (128 sequences, 128-slot rings) cycling
    over `sets` independent ring / q / new-token / output sets (47.5 MB each,
    380 MB for 8, more than the 256 MB MALL holds), so each call's ring comes
    from HBM rather than from the last-level cache.  The calls are enqueued
    back to back and timed together; bytes as for the step's SWA decode."""
    dev = "cuda"
    Bd = len(ctx)
    xs = [synth.decode_inputs(ctx, 0, seed=300 + i, device=dev) for i in range(sets)]
    outs = [(torch.empty((Bd, HQ, DV), dtype=torch.bfloat16, device=dev),
             torch.empty((Bd, HQ), dtype=torch.float32, device=dev)) for _ in range(sets)]
    ctx_d = torch.tensor(ctx, dtype=torch.int32, device=dev)

    def call_all():
        for x, (o, l) in zip(xs, outs):
            B.mimo_attn_decode(dims, 0, x.q, x.k_new, x.v_new, x.k_cache, x.v_cache, None, ctx_d, Bd, max(ctx), 0,
                               x.sink, o, l, None)
    ms = _time_ms(call_all, rounds) / sets
    _, nbytes = decode_stats(ctx, 0)
    del xs, outs
    torch.cuda.empty_cache()
    return {"decode_swa_rotated_rings": {
        "workload": f"SWA decode B={Bd}, 128-slot rings, {sets} independent ring/q/output sets cycled "
                    f"({sets * nbytes / 1e6:.0f} MB, beyond the 256 MB MALL)",
        "ms": ms, "tokens/s": Bd / (ms * 1e-3), "GB/s": nbytes / (ms * 1e-3) / 1e9,
        "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}}


def rope_fused_rows(dims, ga, swa, reps=5):
    """Prefill with the rotary embedding fused in (mimo_attn_prefill_rope: K
    rotated into k_rot with the tokens' cos/sin table, Q rotated as the kernels
    load it) against the separate rotation of q and k (mimo_rope_apply) followed
    by mimo_attn_prefill, on the step's SWA 4 x 8192 and GA 1 x 32768 inputs;
    rotary dims 64, theta 1e4 (SWA) and 5e6 (GA)."""
    dev = "cuda"
    res = {}
    for name, x, lt, nseq, L, theta in (("prefill_rope_swa", swa, 0, 4, 8192, 1e4),
                                        ("prefill_rope_ga", ga, 1, 1, 32768, 5e6)):
        T = x.q.shape[0]
        pos = torch.cat([torch.arange(L, dtype=torch.int32, device=dev)] * nseq)
        out = torch.empty((T, HQ, DV), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((T, HQ), dtype=torch.float32, device=dev)
        krot = torch.empty_like(x.k)
        ws = torch.empty(B.mimo_attn_prefill_rope_workspace_size(dims, T, 64) // 4 + 4, dtype=torch.float32,
                         device=dev)
        fused = lambda: B.mimo_attn_prefill_rope(dims, lt, x.q, x.k, x.v, pos, x.cu_seqlens, nseq, L, T, theta, 64,
                                                 x.sink, out, lse, krot, ws)
        q2, k2 = x.q.clone(), x.k.clone()

        def separate():
            B.mimo_rope_apply(dims, q2, k2, pos, T, theta, 64)
            B.mimo_attn_prefill(dims, lt, q2, k2, x.v, x.cu_seqlens, nseq, L, x.sink, out, lse)
        ms_f, ms_s = _time_ms(fused, reps), _time_ms(separate, reps)
        f = prefill_pairs([L] * nseq, lt) * HQ * FLOP_PER_TRIPLE
        res[name] = {"workload": f"{nseq} x {L} tokens, {'GA' if lt else 'SWA'}, rotary dims 64, theta {theta:g}",
                     "ms": ms_f, "TFLOP/s": f / (ms_f * 1e-3) / 1e12, "separate_rope_then_prefill_ms": ms_s,
                     "saved_ms": ms_s - ms_f}
        if lt == 0:
            res[name]["GB/s"] = T * TOKEN_BYTES / (ms_f * 1e-3) / 1e9
            res[name]["frac_hbm_peak"] = res[name]["GB/s"] / PEAK_HBM_GBPS
        else:
            res[name]["frac_mfma_peak"] = res[name]["TFLOP/s"] / PEAK_BF16_TFLOPS
        del out, lse, krot, ws, q2, k2
    torch.cuda.empty_cache()
    return res


def hybrid_rows(dims, decode_steps=64):
    """The 48-layer hybrid stack (5 SWA : 1 GA), timed end to end: 32 prompts with
    lengths log-uniform in [512, 32768] (seed 0), a varlen prefill of every layer
    (attention + KV append), then `decode_steps` decode steps of all 48 layers
    (attend + append per layer).  There are no weights, so each layer's q/k/v are
    fresh seeded N(0,1) tensors in reused buffers, generated outside the timed
    calls; the sinks are per-layer N(0,1).  Times are HIP-event GPU time of the
    library calls only."""
    from global_attention_mimo_amd.stack import HybridStack, GA as L_GA
    dev = "cuda"
    lengths = synth.hybrid_prompt_lengths(32, seed=0)
    rope_steps = 16  # per RoPE mode, after the plain steps
    st = HybridStack(lengths, decode_steps=decode_steps + 2 * rope_steps, device=dev)
    gen = torch.Generator(device=dev).manual_seed(0)
    sinks = torch.randn((st.num_layers, HQ), generator=gen, device=dev)
    out = torch.empty((st.total, HQ, DV), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((st.total, HQ), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    per_layer = []
    for layer in range(st.num_layers):
        x = synth.prefill_inputs(lengths, seed=1000 + layer, device=dev, with_sink=False)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st.prefill_layer(layer, x.q, x.k, x.v, sinks[layer], out, lse, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        per_layer.append(e0.elapsed_time(e1))
        del x
    lt = st.layer_types
    ga_ms = sum(t for t, l in zip(per_layer, lt) if l == L_GA)
    swa_ms = sum(t for t, l in zip(per_layer, lt) if l != L_GA)
    n_ga = sum(1 for l in lt if l == L_GA)
    f_ga = prefill_pairs(lengths, 1) * HQ * FLOP_PER_TRIPLE * n_ga
    f_swa = prefill_pairs(lengths, 0) * HQ * FLOP_PER_TRIPLE * (len(lt) - n_ga)
    b_swa = st.total * TOKEN_BYTES * (len(lt) - n_ga)
    pre_ms = ga_ms + swa_ms
    # Decode: every step draws all layers' q / k_new / v_new into static buffers
    # first, then runs the 48 layers; the first half of the steps are issued call
    # by call, the second half replay one HIP graph of the step.
    Lyr, Bd = st.num_layers, st.batch
    q = torch.empty((Lyr, Bd, HQ, DQK), dtype=torch.bfloat16, device=dev)
    kn = torch.empty((Lyr, Bd, HKV, DQK), dtype=torch.bfloat16, device=dev)
    vn = torch.empty((Lyr, Bd, HKV, DV), dtype=torch.bfloat16, device=dev)
    dout = torch.empty((Lyr, Bd, HQ, DV), dtype=torch.bfloat16, device=dev)
    dlse = torch.empty((Lyr, Bd, HQ), dtype=torch.float32, device=dev)

    def draw():
        q.copy_(torch.randn(q.shape, generator=gen, device=dev))
        kn.copy_(torch.randn(kn.shape, generator=gen, device=dev))
        vn.copy_(torch.randn(vn.shape, generator=gen, device=dev))

    eager_ms, graph_ms, graph = [], [], None
    for step in range(decode_steps):
        draw()
        if step == decode_steps // 2:
            graph = st.capture_decode_step(q, kn, vn, sinks, dout, dlse)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        if graph is None:
            st.decode_step(q, kn, vn, sinks, dout, dlse, stream)
        else:
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        (eager_ms if graph is None else graph_ms).append(
            (e0.elapsed_time(e1), (time.perf_counter() - t0) * 1e3))
    del graph
    # The same step with q / k_new rotated at their positions (rotary dims 64,
    # theta 5e6): inside the decode calls, or by a separate in-place pass per layer.
    rope_ms = {}
    for mode in ("fused", "separate"):
        st.rope_mode = mode
        graph, times = None, []
        for step in range(rope_steps):
            draw()
            if graph is None:
                graph = st.capture_decode_step(q, kn, vn, sinks, dout, dlse)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        rope_ms[mode] = float(np.mean(times))
        del graph
    # The 48-layer prefill again with RoPE on q and k (positions 0 .. L-1):
    # fused into the prefill (rotated keys appended), or a separate pass first.
    rope_prefill_ms = {}
    for mode in ("fused", "separate"):
        st.rope_mode = mode
        total = 0.0
        for layer in range(st.num_layers):
            x = synth.prefill_inputs(lengths, seed=3000 + layer, device=dev, with_sink=False)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st.prefill_layer(layer, x.q, x.k, x.v, sinks[layer], out, lse, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            total += e0.elapsed_time(e1)
            del x
        rope_prefill_ms[mode] = total
    st.rope_mode = None
    kvb = st.kv_bytes()
    calls = st.num_layers * (1 if st.fused else 2)
    del st, out, lse, dout, dlse
    torch.cuda.empty_cache()
    dec_ms = float(np.mean([g for g, _ in graph_ms]))
    eager_gpu = float(np.mean([g for g, _ in eager_ms]))
    eager_wall = float(np.mean([w for _, w in eager_ms]))
    return {"hybrid_stack": {
        "workload": f"48 layers (5 SWA : 1 GA), 32 prompts log-uniform in [512, 32768] ({sum(lengths)} tokens), "
                    f"prefill then {decode_steps} decode steps; attention + KV append per layer",
        "prefill_ms": pre_ms, "prefill_tokens/s": sum(lengths) / (pre_ms * 1e-3),
        "prefill_TFLOP/s": (f_ga + f_swa) / (pre_ms * 1e-3) / 1e12,
        "prefill_ga_layers_ms": ga_ms, "prefill_ga_TFLOP/s": f_ga / (ga_ms * 1e-3) / 1e12,
        "prefill_ga_frac_mfma_peak": f_ga / (ga_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "prefill_swa_layers_ms": swa_ms, "prefill_swa_GB/s": b_swa / (swa_ms * 1e-3) / 1e9,
        "prefill_swa_frac_hbm_peak": b_swa / (swa_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "decode_step_ms": dec_ms, "decode_tokens/s": Bd / (dec_ms * 1e-3),
        "decode_step_note": f"HIP-graph replay of the whole step ({calls} library calls + context advance), mean of "
                            f"{len(graph_ms)} steps; the first {len(eager_ms)} steps issued call by call took "
                            f"{eager_gpu:.3f} ms on the GPU clock and {eager_wall:.3f} ms host wall time",
        "prefill_rope_fused_ms": rope_prefill_ms["fused"], "prefill_rope_separate_ms": rope_prefill_ms["separate"],
        "decode_step_rope_fused_ms": rope_ms["fused"], "decode_step_rope_separate_ms": rope_ms["separate"],
        "decode_step_rope_note": f"the step with RoPE (rotary dims 64, theta 5e6, positions = contexts) on each "
                                 f"layer's q and k_new, HIP-graph replay, mean of {rope_steps} steps each: fused "
                                 f"(mimo_attn_decode_append_rope) against mimo_rope_apply + mimo_attn_decode_append; "
                                 f"prefill_rope_*: all 48 layers' prefill + append with RoPE at positions 0..L-1, "
                                 f"fused (mimo_attn_prefill_rope, k_rot appended) against mimo_rope_apply first",
        "kv_cache_bytes": kvb["hybrid"], "kv_cache_bytes_all_ga": kvb["all_ga"]}}


def copy_calibration(dev):
    """A plain 1 GiB device-to-device copy, for scaling the HBM byte counters of
    a profiled run (its FETCH_SIZE / WRITE_SIZE against the known bytes)."""
    src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)  # reads 1 GiB, writes 1 GiB
    torch.cuda.synchronize()
    del src, dst
    log("copy calibration: 1 GiB device-to-device copy done")


def _time_ms(call, reps):
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def device_context():
    """The box's own figures next to the spec-sheet peaks: CU count and a measured
    device-to-device copy rate (read + write bytes per second, 2 GiB buffers)."""
    props = torch.cuda.get_device_properties(0)
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    clock_mhz = _hip_attribute("hipDeviceAttributeClockRate", 5) / 1e3  # kHz -> MHz
    cus = props.multi_processor_count
    # 4 SIMDs per CU, 1024 dense bf16 flops per SIMD per clock (v_mfma_f32_32x32x16_bf16: 32768 flops in 32 clocks).
    peak_from_clock = cus * 4 * 1024 * clock_mhz * 1e6 / 1e12 if clock_mhz > 0 else None
    return {"name": props.name, "compute_units": cus, "max_clock_MHz": clock_mhz,
            "bf16_dense_peak_from_clock_TFLOPs": peak_from_clock,
            "copy_GBps": 2 * n / (ms * 1e-3) / 1e9,
            "note": "copy_GBps: torch device-to-device copy of 2 GiB, read + write bytes; peaks used are the spec "
                    "sheet's (2500 TFLOP/s bf16 dense, 8000 GB/s HBM)"}


def _hip_attribute(name, value):
    """hipDeviceGetAttribute(value) on device 0 through the HIP runtime torch loaded; 0 if unavailable."""
    import ctypes
    for lib in ("libamdhip64.so", "libamdhip64.so.7", "libamdhip64.so.6"):
        try:
            hip = ctypes.CDLL(lib)
            break
        except OSError:
            hip = None
    if hip is None:
        return 0
    out = ctypes.c_int(0)
    return out.value if hip.hipDeviceGetAttribute(ctypes.byref(out), value, 0) == 0 else 0


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(swa, ga, dga, dswa, ctx, gpu, sample_s=4.0):
    """The fp64 oracle, as it stands, timed per configuration on the host cores,
    next to the GPU figure of the same configuration (`gpu`: name -> dict).
    Configs 1, 2 and 4-SWA run in full; configs 3, 4-GA and 5 run on a sample of
    about `sample_s` seconds each and their time is extrapolated by algorithmic
    flops (labelled as such)."""
    import oracle
    orc = oracle.get()
    nth = orc.default_threads()
    scale = float(np.float32(synth.SOFTMAX_SCALE))
    rng = np.random.default_rng(0)
    rows, tot_flops, tot_s = {}, 0, 0.0

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def record(name, flops_done, secs, flops_config, coverage):
        nonlocal tot_flops, tot_s
        tot_flops += flops_done
        tot_s += secs
        est = secs * flops_config / flops_done
        r = {"coverage": coverage, "oracle_s": secs, "oracle_GFLOP_s": flops_done / secs / 1e9,
             "oracle_config_s": est, "oracle_config_s_kind": "measured" if flops_done == flops_config else
             "extrapolated by algorithmic flops"}
        if name in gpu and gpu[name].get("ms"):
            r["gpu_ms"] = gpu[name]["ms"]
            r["gpu_speedup"] = est * 1e3 / gpu[name]["ms"]
        rows[name] = r
        log(f"cpu_baseline {name}: {coverage}, {secs:.1f} s")

    # 1: SWA prefill 1 x 256, whole configuration.
    x1 = synth.prefill_inputs([256], seed=0)
    b1 = [synth.bf16_bits(t) for t in (x1.q, x1.k, x1.v)]
    f1 = prefill_pairs([256], 0) * HQ * FLOP_PER_TRIPLE
    s1 = timed(lambda: orc.prefill(*b1, x1.cu_seqlens.numpy(), layer_type=0, scale=scale, sink=x1.sink.numpy(),
                                   nthreads=nth))
    record("config1_swa_prefill_1x256", f1, s1, f1, "full")
    # 2: SWA prefill 4 x 8192, whole configuration.
    b2 = [synth.bf16_bits(t) for t in (swa.q, swa.k, swa.v)]
    cu2, sk2 = swa.cu_seqlens.cpu().numpy(), swa.sink.cpu().numpy()
    f2 = prefill_pairs([8192] * 4, 0) * HQ * FLOP_PER_TRIPLE
    s2 = timed(lambda: orc.prefill(*b2, cu2, layer_type=0, scale=scale, sink=sk2, nthreads=nth))
    record("config2_swa_prefill_4x8192", f2, s2, f2, "full (32768 tokens)")
    del b2
    # 3: GA prefill 1 x 32768: random query rows, 16 at a time, for about `sample_s` seconds.
    b3 = [synth.bf16_bits(t) for t in (ga.q, ga.k, ga.v)]
    order3 = rng.permutation(32768)
    f3s, s3, n3 = 0, 0.0, 0
    while s3 < sample_s and n3 < 2048:
        r3 = np.sort(order3[n3:n3 + 16])
        s3 += timed(lambda: orc.prefill(*b3, ga.cu_seqlens.cpu().numpy(), layer_type=1, scale=scale,
                                        sink=ga.sink.cpu().numpy(), rows=r3, nthreads=nth))
        f3s += int((r3 + 1).sum()) * HQ * FLOP_PER_TRIPLE
        n3 += 16
    record("config3_ga_prefill_1x32768", f3s, s3, prefill_pairs([32768], 1) * HQ * FLOP_PER_TRIPLE,
           f"{n3} random query rows of 32768")
    del b3
    # 4-GA: whole sequences of the 128, in random order, for about `sample_s` seconds.
    base = dga.kv_base.cpu().numpy()
    pick = rng.permutation(len(ctx))
    f4s, s4, n4 = 0, 0.0, 0
    for b in pick:
        if s4 >= sample_s:
            break
        c = int(ctx[b])
        kc = synth.bf16_bits(dga.k_cache[base[b]:base[b] + c])
        vc = synth.bf16_bits(dga.v_cache[base[b]:base[b] + c])
        args = [synth.bf16_bits(t[b:b + 1]) for t in (dga.q, dga.k_new, dga.v_new)]
        s4 += timed(lambda: orc.decode(*args, kc, vc, np.array([c], np.int32), layer_type=1, scale=scale,
                                       sink=dga.sink.cpu().numpy(), kv_base=np.zeros(1, np.int64), nthreads=nth))
        f4s += (c + 1) * HQ * FLOP_PER_TRIPLE
        n4 += 1
    record("config4_ga_decode_b128", f4s, s4, sum(int(c) + 1 for c in ctx) * HQ * FLOP_PER_TRIPLE,
           f"{n4} of the {len(ctx)} sequences, whole")
    # 4-SWA: all 128 sequences over the ring.
    a5 = [synth.bf16_bits(t) for t in (dswa.q, dswa.k_new, dswa.v_new, dswa.k_cache, dswa.v_cache)]
    f4w = len(ctx) * W * HQ * FLOP_PER_TRIPLE
    s4w = timed(lambda: orc.decode(*a5, np.asarray(ctx, np.int32), layer_type=0, scale=scale,
                                   sink=dswa.sink.cpu().numpy(), nthreads=nth))
    record("config4_swa_decode_b128", f4w, s4w, f4w, f"full ({len(ctx)} sequences)")
    # 5: the 48-layer stack: 24 rows of one prompt of median length per layer type, extrapolated to the
    # stack's prefill flops (8 GA + 40 SWA layers) and 64 decode steps of all 48 layers.
    lengths = synth.hybrid_prompt_lengths(32, seed=0)
    Lm = int(np.median(lengths))
    x5 = synth.prefill_inputs([Lm], seed=1000)
    b5 = [synth.bf16_bits(t) for t in (x5.q, x5.k, x5.v)]
    order5 = rng.permutation(Lm)
    f5s, s5, n5 = 0, 0.0, 0
    while s5 < sample_s and n5 < Lm:
        r5 = np.sort(order5[n5:n5 + 24])
        for lt in (0, 1):
            s5 += timed(lambda: orc.prefill(*b5, x5.cu_seqlens.numpy(), layer_type=lt, scale=scale,
                                            sink=x5.sink.numpy(), rows=r5, nthreads=nth))
            f5s += int(np.minimum(r5 + 1, W if lt == 0 else 1 << 40).sum()) * HQ * FLOP_PER_TRIPLE
        n5 += len(r5)
    f5 = (8 * prefill_pairs(lengths, 1) + 40 * prefill_pairs(lengths, 0)) * HQ * FLOP_PER_TRIPLE
    f5 += sum(8 * sum(L + s + 1 for L in lengths) + 40 * len(lengths) * W for s in range(64)) * HQ * FLOP_PER_TRIPLE
    record("config5_hybrid_stack", f5s, s5, f5, f"{n5} query rows of a {Lm}-token prompt per layer type")
    return {"value": tot_flops / tot_s / 1e12, "unit": "TFLOP/s", "cores": nth, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"per configuration below; {tot_flops / 1e9:.1f} GFLOP of fp64 oracle work in {tot_s:.1f} s "
                      f"on {nth} host threads (configs 1, 2 and 4-SWA whole, 3, 4-GA and 5 sampled)",
            "configs": rows}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the rows timed apart from the step (chunked prefill, paged and FP8 pools, "
                         "backward, RoPE, the 48-layer hybrid stack)")
    ap.add_argument("--split", type=int, default=0, help="GA decode split (keys per workgroup), 0 = default")
    ap.add_argument("--no-hybrid", action="store_true", help="skip the 48-layer hybrid stack")
    ap.add_argument("--hybrid-only", action="store_true",
                    help="time only the 48-layer hybrid stack (prefill + decode steps) and print its JSON")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device copy (a known-size reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this path runs on one MI355X with no collectives)", file=sys.stderr)
        sys.exit(2)
    headroom = args.steps + args.warmup + 1
    dev = "cuda"
    torch.cuda.set_device(0)
    if args.hybrid_only:
        if args.copy_calibration:
            copy_calibration(dev)
        log("hybrid stack: 48-layer prefill and decode")
        print(json.dumps({"metric": METRIC, "n_gpus": 1, "data": "synthetic", **hybrid_rows(B.make_dims())}),
              flush=True)
        return
    log("generating inputs on the device")
    swa = synth.prefill_inputs([8192] * 4, seed=0, device=dev)
    ga = synth.prefill_inputs([32768], seed=0, device=dev)
    ctx0 = synth.long_context_lengths(128, 4096, 262144, seed=0)
    dga = synth.decode_inputs(ctx0, 1, seed=0, device=dev, headroom=headroom)
    dswa = synth.decode_inputs(ctx0, 0, seed=0, device=dev)
    T_swa, T_ga = swa.q.shape[0], ga.q.shape[0]
    out_swa = torch.empty((T_swa, HQ, DV), dtype=torch.bfloat16, device=dev)
    lse_swa = torch.empty((T_swa, HQ), dtype=torch.float32, device=dev)
    out_ga = torch.empty((T_ga, HQ, DV), dtype=torch.bfloat16, device=dev)
    lse_ga = torch.empty((T_ga, HQ), dtype=torch.float32, device=dev)
    Bd = len(ctx0)
    out_d = torch.empty((2, Bd, HQ, DV), dtype=torch.bfloat16, device=dev)
    lse_d = torch.empty((2, Bd, HQ), dtype=torch.float32, device=dev)
    ctx_ga = dga.ctx_lens.clone()
    ctx_swa = dswa.ctx_lens.clone()
    max_ctx = max(ctx0) + headroom
    dims = B.make_dims()
    ws_bytes = B.mimo_attn_decode_workspace_size(dims, 1, Bd, max_ctx, args.split)
    ws = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device=dev)
    cu_dec = torch.arange(Bd + 1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready: GA pool {dga.k_cache.numel() * 2 / 1e9 + dga.v_cache.numel() * 2 / 1e9:.1f} GB, "
        f"workspace {ws_bytes / 1e6:.0f} MB")

    if args.copy_calibration:
        copy_calibration(dev)

    stream = torch.cuda.current_stream()
    names = ["prefill_swa", "prefill_ga", "decode_swa", "append_swa", "decode_ga", "append_ga", "ctx_advance"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        B.mimo_attn_prefill(dims, 0, swa.q, swa.k, swa.v, swa.cu_seqlens, 4, 8192, swa.sink, out_swa, lse_swa, stream)
        mark(1)
        B.mimo_attn_prefill(dims, 1, ga.q, ga.k, ga.v, ga.cu_seqlens, 1, 32768, ga.sink, out_ga, lse_ga, stream)
        mark(2)
        B.mimo_attn_decode(dims, 0, dswa.q, dswa.k_new, dswa.v_new, dswa.k_cache, dswa.v_cache, None, ctx_swa, Bd,
                           max_ctx, 0, dswa.sink, out_d[0], lse_d[0], None, stream)
        mark(3)
        B.mimo_kv_append(dims, 0, dswa.k_new, dswa.v_new, cu_dec, ctx_swa, Bd, Bd, dswa.k_cache, dswa.v_cache, None,
                         None, stream)
        mark(4)
        B.mimo_attn_decode(dims, 1, dga.q, dga.k_new, dga.v_new, dga.k_cache, dga.v_cache, dga.kv_base, ctx_ga, Bd,
                           max_ctx, args.split, dga.sink, out_d[1], lse_d[1], ws, stream)
        mark(5)
        B.mimo_kv_append(dims, 1, dga.k_new, dga.v_new, cu_dec, ctx_ga, Bd, Bd, dga.k_cache, dga.v_cache,
                         dga.kv_base, dga.kv_capacity, stream)
        mark(6)
        ctx_ga.add_(1)
        ctx_swa.add_(1)
        mark(7)

    dev_ctx = device_context()
    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    # The timed steps start from the contexts the warmup left.
    ctx_host = [np.asarray(ctx0) + args.warmup + s for s in range(args.steps)]
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall:.3f} s")

    per = {n: [] for n in names}
    for ev in events:
        for i, n in enumerate(names):
            per[n].append(ev[i].elapsed_time(ev[i + 1]))  # ms
    avg = {n: float(np.mean(v)) for n, v in per.items()}
    step_ms = wall * 1e3 / args.steps

    f_pswa = prefill_pairs([8192] * 4, 0) * HQ * FLOP_PER_TRIPLE
    f_pga = prefill_pairs([32768], 1) * HQ * FLOP_PER_TRIPLE
    b_pswa, b_pga = T_swa * TOKEN_BYTES, T_ga * TOKEN_BYTES
    dec = {lt: [decode_stats(c, lt) for c in ctx_host] for lt in (0, 1)}
    f_dswa = float(np.mean([d[0] for d in dec[0]]))
    b_dswa = float(np.mean([d[1] for d in dec[0]]))
    f_dga = float(np.mean([d[0] for d in dec[1]]))
    b_dga = float(np.mean([d[1] for d in dec[1]]))
    app_bytes = 2 * Bd * KV_TOKEN_BYTES
    total_flops = f_pswa + f_pga + f_dswa + f_dga
    value = total_flops / (step_ms * 1e-3) / 1e12

    def tf(f, ms):
        return f / (ms * 1e-3) / 1e12

    def gbs(b, ms):
        return b / (ms * 1e-3) / 1e9

    breakdown = {
        "prefill_swa": {"ms": avg["prefill_swa"], "TFLOP/s": tf(f_pswa, avg["prefill_swa"]),
                        "GB/s": gbs(b_pswa, avg["prefill_swa"]),
                        "frac_hbm_peak": gbs(b_pswa, avg["prefill_swa"]) / PEAK_HBM_GBPS,
                        "frac_mfma_peak": tf(f_pswa, avg["prefill_swa"]) / PEAK_BF16_TFLOPS},
        "prefill_ga": {"ms": avg["prefill_ga"], "TFLOP/s": tf(f_pga, avg["prefill_ga"]),
                       "frac_mfma_peak": tf(f_pga, avg["prefill_ga"]) / PEAK_BF16_TFLOPS},
        "decode_swa": {"ms": avg["decode_swa"], "tokens/s": Bd / (avg["decode_swa"] * 1e-3),
                       "GB/s": gbs(b_dswa, avg["decode_swa"]),
                       "frac_hbm_peak": gbs(b_dswa, avg["decode_swa"]) / PEAK_HBM_GBPS},
        "decode_ga": {"ms": avg["decode_ga"], "tokens/s": Bd / (avg["decode_ga"] * 1e-3),
                      "GB/s": gbs(b_dga, avg["decode_ga"]),
                      "frac_hbm_peak": gbs(b_dga, avg["decode_ga"]) / PEAK_HBM_GBPS},
        "append_swa": {"ms": avg["append_swa"], "GB/s": gbs(app_bytes / 2, avg["append_swa"])},
        "append_ga": {"ms": avg["append_ga"], "GB/s": gbs(app_bytes / 2, avg["append_ga"])},
        "ctx_advance": {"ms": avg["ctx_advance"]},
    }
    # Dominant kernel of the step: the GA prefill launch (MFMA-bound).
    roof = {"kernel": "prefill_kernel<GA>", "bound": "mfma", "achieved": tf(f_pga, avg["prefill_ga"]),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": tf(f_pga, avg["prefill_ga"]) / PEAK_BF16_TFLOPS,
            "traffic": measured_traffic(), "traffic_unit": "bytes per launch (HBM read + write)",
            "algorithmic_bytes": b_pga}
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/k/v, N(0,1) fp32 sinks; no weights involved)",
        "config": {"workload": "one hybrid-attention pass: SWA prefill 4x8192 + GA prefill 1x32768 + decode step "
                               "B=128 ctx~U[4096,262144] (SWA ring 128 slots + GA bf16 pool, attend then append)",
                   "heads": "64q/4kv", "head_dim_qk": DQK, "head_dim_v": DV, "sliding_window": W,
                   "global_batch": {"prefill_swa": 4, "prefill_ga": 1, "decode": Bd},
                   "seq_len": {"prefill_swa": 8192, "prefill_ga": 32768, "decode_ctx_mean": float(np.mean(ctx0))},
                   "parallelism": "none (1 GPU)"},
        "breakdown": breakdown,
        "roofline": roof,
        "device": dev_ctx,
    }
    # Config 1 (the small parity configuration, SWA prefill 1 x 256): latency, no roofline target.
    x1 = synth.prefill_inputs([256], seed=0, device=dev)
    o1 = torch.empty((256, HQ, DV), dtype=torch.bfloat16, device=dev)
    l1 = torch.empty((256, HQ), dtype=torch.float32, device=dev)
    small_ms = _time_ms(lambda: B.mimo_attn_prefill(dims, 0, x1.q, x1.k, x1.v, x1.cu_seqlens, 1, 256, x1.sink, o1, l1),
                        20)
    res["config1_swa_prefill_1x256"] = {"ms": small_ms,
                                        "TFLOP/s": tf(prefill_pairs([256], 0) * HQ * FLOP_PER_TRIPLE, small_ms)}
    if not args.no_next_rows:
        res["next_rows"] = {**chunk_rows(dims, ga, swa), **paged_rows(dims, dga, ctx_ga, max_ctx, ws, ga),
                            **fp8_rows(dims, dga, ctx_ga, max_ctx, ws, ga),
                            **backward_rows(dims, ga, swa, out_ga, lse_ga, out_swa, lse_swa),
                            **rope_rows(dims, ga), **rope_fused_rows(dims, ga, swa),
                            **swa_decode_rotated_rows(dims, ctx0)}
    if not args.no_next_rows and not args.no_hybrid:
        log("hybrid stack: 48-layer prefill and decode")
        res["hybrid_stack"] = hybrid_rows(dims)["hybrid_stack"]
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample (cpu_baseline)")
        gpu = {"config2_swa_prefill_4x8192": breakdown["prefill_swa"],
               "config3_ga_prefill_1x32768": breakdown["prefill_ga"],
               "config4_ga_decode_b128": breakdown["decode_ga"], "config4_swa_decode_b128": breakdown["decode_swa"],
               "config1_swa_prefill_1x256": {"ms": small_ms}}
        if "hybrid_stack" in res:
            h = res["hybrid_stack"]
            gpu["config5_hybrid_stack"] = {"ms": h["prefill_ms"] + 64 * h["decode_step_ms"]}
        res["cpu_baseline"] = cpu_baseline(swa, ga, dga, dswa, ctx0, gpu)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
