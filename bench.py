#!/usr/bin/env python3
"""Benchmark of one decode/verify attention call through the C ABI (librattn).

A step is one ``rattn_decode`` call: one attention layer for one decode (or verify)
step over the whole batch, i.e. the split-KV kernel and, when the planner splits the
key range, the log-sum-exp combine. Inputs are synthetic, seeded, and resident in HBM
before the timed region starts.

Default workload: full-context layer decode, 48 query / 8 KV heads, head size 128,
batch 1, one query row, 100,000 keys in a bf16 cache paged by 16 tokens (random page
permutation), bias table of 131,072 distances (page 1, "vLLM supports Inkling 2 Small",
section on vLLM's optimisations: batch-1 decode at 100K context).

Cache hygiene: the inputs are cloned into enough copies that the steps rotate over at
least 1 GiB, four times the 256 MiB Infinity Cache, so every step streams its K/V from
HBM. Three passes of K steps each:
  1. back to back between two device synchronisations, launched as a caller would:
     the reported µs/step;
  2. the library launches each step's kernels with HIP events that the runtime stamps
     with the kernel's own start and end: the per-kernel durations of the roofline (the
     stamping adds launch overhead, so this pass is not the figure);
  3. each step between a pair of events on the launch stream: the median, p10 and p90
     of single steps.

Output: one JSON line (rank 0, N = 1) with the step time, the achieved HBM bandwidth
over the algorithmic bytes, the roofline of the dominant kernel and the CPU oracle's
time on the host cores.
"""

import argparse
import ctypes
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn µs/step + achieved HBM GB/s; 48q/8kv GQA, d=128, 100K ctx, b=1"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (no sparsity)
CACHE_EVICT_BYTES = 1 << 30     # rotate over at least this many input bytes
PLAN_REPS = 20                  # host planning calls timed (rattn_plan + rattn_free)
KERNEL_SOURCES = ("csrc/device_common.h", "csrc/split_kv.h", "csrc/internal.h",
                  "csrc/planner.cpp")   # what decides the split kernel and its launch

WORKLOADS = {
    "full_100k": "full-context layer decode, 48q/8kv, d=128, batch 1, 1 row, 100,000 keys, "
                 "bf16 paged KV (page 16), Dmax=131071",
    "window_b1": "sliding-window (W=1024) layer decode, 48q/8kv, d=128, batch 1, 1 row, "
                 "seq_lens U[2048,32768], bf16 paged KV (page 16)",
    "window_b16": "sliding-window (W=1024) layer decode, 48q/8kv, d=128, batch 16, 1 row, "
                  "seq_lens U[2048,32768], bf16 paged KV (page 16)",
    "window_b64": "sliding-window (W=1024) layer decode, 48q/8kv, d=128, batch 64, 1 row, "
                  "seq_lens U[2048,32768], bf16 paged KV (page 16)",
    "window_verify_b16": "speculative verify, 8 causal rows, sliding-window (W=1024) layer, 48q/8kv, "
                         "d=128, batch 16, seq_lens U[2048,32768], bf16 paged KV (page 16)",
    "verify_b16": "speculative verify, 8 causal rows, 48q/8kv, d=128, batch 16, full layer, "
                  "seq_lens log-uniform [32768,262144], bf16 paged KV (page 16)",
    "verify4_100k": "single-user speculative step, 4 causal rows, 48q/8kv, d=128, batch 1, "
                    "100,000 keys, full layer, bf16 paged KV (page 16)",
    "verify3_b16": "speculative verify, 3 causal rows (2 drafts), 48q/8kv, d=128, batch 16, "
                   "full layer, seq_lens log-uniform [32768,262144], bf16 paged KV (page 16)",
    "fp8_1m": "full-context layer decode, 48q/8kv, d=128, batch 1, 1 row, 1,048,576 keys, "
              "E4M3 KV + fp32 per-token-per-head scales, paged (page 64)",
    "tiny": "full-context decode, 6q/1kv, d=128, batch 1, 1 row, 2048 keys, contiguous bf16",
    "v1_full_decode": "full-context layer decode, 64q/8kv, d=128, batch 1, 1 row, 100,000 keys, "
                      "bf16 paged KV (page 16)",
    "v1_window_decode": "sliding-window (W=512) layer decode, 64q/16kv, d=128, batch 16, 1 row, "
                        "seq_lens U[2048,32768], bf16 paged KV (page 16)",
    "v1_full_verify": "verify, 8 causal rows, 64q/8kv, d=128, batch 4, full layer, seq_lens "
                      "log-uniform [32768,262144], bf16 paged KV (page 16)",
    "v1_window_verify": "verify, 9 causal rows, 64q/16kv, d=128, batch 16, W=512, seq_lens "
                        "U[2048,32768], bf16 paged KV (page 16)",
    "v1_full_mtp9": "verify of a 9-token MTP step, 9 causal rows, 64q/8kv, d=128, batch 4, "
                    "full layer, seq_lens log-uniform [32768,262144], bf16 paged KV (page 16)",
    "v1_full_mtp9_varlen": "verify of a 9-token MTP step with 1..9 rows per sequence (seeded), "
                           "64q/8kv, d=128, batch 4, full layer, seq_lens log-uniform "
                           "[32768,262144], bf16 paged KV (page 16)",
    "tp4_100k": "one GPU's TP4 share of the full-context layer: 12q/2kv, d=128, batch 1, "
                "1 row, 100,000 keys, bf16 paged KV (page 16)",
    "tp8_100k": "one GPU's TP8 share of the full-context layer: 6q/1kv, d=128, batch 1, "
                "1 row, 100,000 keys, bf16 paged KV (page 16)",
    "prefill_8x2k": "chunked prefill: 8 sequences, a chunk of 2048 query tokens each at "
                    "100,000 keys (the chunk included), 48q/8kv, d=128, causal, bf16 paged "
                    "KV (page 16)",
    "prefill_8x2k_fp8": "chunked prefill: 8 sequences, a chunk of 2048 query tokens each at "
                        "100,000 keys (the chunk included), 48q/8kv, d=128, causal, E4M3 KV + "
                        "fp32 per-token-per-head scales, paged (page 64)",
    "prefill_4x2k_g8": "chunked prefill: 4 sequences, a chunk of 2048 query tokens each at "
                       "32,768 keys (the chunk included), 64q/8kv, d=128, causal, bf16 paged "
                       "KV (page 16)",
    "prefill_4x2k_g4": "chunked prefill: 4 sequences, a chunk of 2048 query tokens each at "
                       "32,768 keys (the chunk included), 64q/16kv, d=128, causal, bf16 paged "
                       "KV (page 16)",
    "verify_b16_fp8": "speculative verify, 8 causal rows, 48q/8kv, d=128, batch 16, full layer, "
                      "seq_lens log-uniform [32768,262144], E4M3 KV + fp32 per-token-per-head "
                      "scales, paged (page 64)",
    "decode_b16_fp8": "full-context layer decode, 48q/8kv, d=128, batch 16, 1 row, seq_lens "
                      "log-uniform [32768,262144], E4M3 KV + fp32 per-token-per-head scales, "
                      "paged (page 64)",
    "verify3_b16_8k": "speculative verify, 3 causal rows (2 drafts), 48q/8kv, d=128, batch 16, "
                      "full layer, seq_lens log-uniform [2048,8191], bf16 paged KV (page 16)",
    "verify3_b16_fp8": "speculative verify, 3 causal rows (2 drafts), 48q/8kv, d=128, batch 16, "
                       "full layer, seq_lens log-uniform [32768,262144], E4M3 KV + fp32 "
                       "per-token-per-head scales, paged (page 64)",
    "verify_b16_varlen": "speculative verify with 1..8 rows per sequence (seeded), 48q/8kv, "
                         "d=128, batch 16, full layer, seq_lens log-uniform [32768,262144], "
                         "bf16 paged KV (page 16)",
}


def say(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def settle(ms, mib=256, n=4096):
    """Untimed load ahead of the warm-up steps: n x n x n bf16 matrix products and
    device-to-device copies of a scratch buffer of mib MiB, interleaved, for at least ms
    milliseconds. A GPU that has sat idle (input generation, planning) starts at low
    clocks and takes a few hundred milliseconds of load to reach its steady ones, the
    matrix cores' clock the slowest; a handful of short warm-up steps is not that long.
    None of this work touches the attention path or its inputs, and its buffers pass
    through the caches after the inputs, so it leaves no cache advantage behind. Returns
    the milliseconds spent."""
    import torch
    if ms <= 0:
        return 0.0
    a = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    x = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    y = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            b.copy_(a)
            torch.mm(x, y)
        torch.cuda.synchronize()
    spent = (time.perf_counter() - t0) * 1e3
    del a, b, x, y
    return spent


def kernel_digest():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_verify_amd", rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload, digest):
    """HBM bytes per split-kernel launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_split_kv_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_digest") != digest or "hbm_bytes_per_launch" not in vals:
        return None
    return float(vals["hbm_bytes_per_launch"])


def copy_probe(mib, reps):
    """A plain device-to-device copy of known size, for scaling the HBM counters."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "reps": reps}), flush=True)


def cpu_baseline(case_cpu, tr, budget_s, rows=None, q_packed=None, cu=None):
    """Time the fp64 oracle on the host cores, (sequence, KV head) unit by unit in
    order, repeating whole passes over the step until ``budget_s`` is spent (a pass cut
    short by the budget is scaled to the whole step by its visible-key work)."""
    import numpy as np
    import torch
    import oracle
    from decode_attention_verify_amd import accounting
    try:
        from threadpoolctl import threadpool_info
        blas = [p.get("num_threads", 1) for p in threadpool_info()
                if p.get("user_api") == "blas"]
        cores = max(blas) if blas else 1
    except Exception:                                   # threadpoolctl missing
        cores = 1
    a = case_cpu
    sp = a.spec
    tv = torch.uint16 if a.k_cache.dtype == torch.bfloat16 else torch.uint8
    q = a.q.view(torch.uint16).numpy()
    kc = a.k_cache.view(tv).numpy()
    vc = a.v_cache.view(tv).numpy()
    pt, sl, bias = a.page_table.numpy(), a.seq_lens.numpy(), a.bias.numpy()
    ks = None if a.k_scale is None else a.k_scale.numpy()
    vs = None if a.v_scale is None else a.v_scale.numpy()
    G = sp.num_q_heads // sp.num_kv_heads
    lens = [int(x) for x in sl]
    nrows = [sp.n_rows] * sp.batch if rows is None else rows
    unit_work = [accounting.rows_keys(L, n, sp.window) for L, n in zip(lens, nrows)]
    total_work = sum(unit_work) * sp.num_kv_heads
    if rows is None:
        out = np.full((sp.batch, sp.n_rows, sp.num_q_heads, sp.head_dim), np.nan)
        lse = np.full((sp.batch, sp.n_rows, sp.num_q_heads), np.nan)
    else:
        qp = q_packed.view(torch.uint16).numpy()
        cun = cu.numpy()
        out = np.full((qp.shape[0], sp.num_q_heads, sp.head_dim), np.nan)
        lse = np.full((qp.shape[0], sp.num_q_heads), np.nan)
    done_work = 0
    units = 0
    t0 = time.perf_counter()
    while True:
        for b in range(sp.batch):
            for g in range(sp.num_kv_heads):
                hs = slice(g * G, (g + 1) * G)
                if rows is None:
                    o, l = oracle.relative_attention(
                        q, kc, vc, pt, sl, bias, n_query_rows=sp.n_rows, window=sp.window,
                        dmax=sp.dmax, softmax_scale=a.softmax_scale, k_scale=ks, v_scale=vs,
                        batches=[b], kv_heads=[g])
                    out[b, :, hs] = o[b, :, hs]
                    lse[b, :, hs] = l[b, :, hs]
                else:
                    o, l = oracle.relative_attention_varlen(
                        qp, cun, kc, vc, pt, sl, bias, window=sp.window, dmax=sp.dmax,
                        softmax_scale=a.softmax_scale, k_scale=ks, v_scale=vs, batches=[b],
                        kv_heads=[g])
                    rs = slice(int(cun[b]), int(cun[b + 1]))
                    out[rs, hs] = o[rs, hs]
                    lse[rs, hs] = l[rs, hs]
                done_work += unit_work[b]
                units += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    secs = time.perf_counter() - t0
    steps = done_work / total_work
    us_step = secs / steps * 1e6
    return {
        "value": us_step,
        "unit": "us/step",
        "cores": cores,
        "kind": "oracle",
        "sample": "%.2f passes over the whole step (%d (sequence, KV head) units of %d per "
                  "pass) in %.1f s; fp64 numpy, BLAS threads=%d, elementwise work "
                  "single-threaded" % (steps, units, sp.batch * sp.num_kv_heads, secs, cores),
        "GBps": tr.total / (us_step * 1e-6) / 1e9,
    }, out, lse


def cpu_baseline_rows(case_cpu, tr, budget_s, block=32):
    """The oracle on the host cores for a chunk of many rows: blocks of `block` rows of
    one (sequence, KV head), each attended as the last rows of the sequence cut after
    them (the same rows of a shorter sequence), in a seeded random order until
    ``budget_s`` is spent; scaled to the whole step by visible-key work."""
    import numpy as np
    import torch
    import oracle
    from decode_attention_verify_amd import accounting
    try:
        from threadpoolctl import threadpool_info
        blas = [p.get("num_threads", 1) for p in threadpool_info()
                if p.get("user_api") == "blas"]
        cores = max(blas) if blas else 1
    except Exception:
        cores = 1
    a = case_cpu
    sp = a.spec
    n, G = sp.n_rows, sp.num_q_heads // sp.num_kv_heads
    tv = torch.uint16 if a.k_cache.dtype == torch.bfloat16 else torch.uint8
    kc, vc = a.k_cache.view(tv).numpy(), a.v_cache.view(tv).numpy()
    ks = None if a.k_scale is None else a.k_scale.numpy()
    vs = None if a.v_scale is None else a.v_scale.numpy()
    q = a.q.view(torch.uint16).numpy()
    lens = [int(x) for x in a.seq_lens]
    total_work = sum(accounting.rows_keys(L, n, sp.window) for L in lens) * sp.num_kv_heads
    out = np.full((sp.batch, n, sp.num_q_heads, sp.head_dim), np.nan)
    lse = np.full((sp.batch, n, sp.num_q_heads), np.nan)
    rng = np.random.default_rng(0)
    done, blocks = 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b = int(rng.integers(0, sp.batch))
        g = int(rng.integers(0, sp.num_kv_heads))
        r0 = int(rng.integers(0, n // block)) * block
        r1 = min(r0 + block, n)
        L_cut = lens[b] - (n - r1)
        o, l = oracle.relative_attention(
            q[b:b + 1, r0:r1], kc, vc, a.page_table[b:b + 1].numpy(), np.array([L_cut]),
            a.bias.numpy(), n_query_rows=r1 - r0, window=sp.window, dmax=sp.dmax,
            softmax_scale=a.softmax_scale, k_scale=ks, v_scale=vs, kv_heads=[g])
        hs = slice(g * G, (g + 1) * G)
        out[b, r0:r1, hs] = o[0, :, hs]
        lse[b, r0:r1, hs] = l[0, :, hs]
        done += accounting.rows_keys(L_cut, r1 - r0, sp.window)
        blocks += 1
    secs = time.perf_counter() - t0
    us_step = secs * total_work / done * 1e6
    return {
        "value": us_step,
        "unit": "us/step",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d blocks of %d rows of one (sequence, KV head), %.4f of the step's "
                  "visible-key work, in %.1f s, scaled to the whole step; fp64 numpy, BLAS "
                  "threads=%d" % (blocks, block, done / total_work, secs, cores),
        "TFLOPs": tr.flops / (us_step * 1e-6) / 1e12,
    }, out, lse


def read_probe(lib, case, sp, fp8, num_cus, reps=8, seed=0):
    """The read rate the split kernel's access pattern reaches on this device: buffers of
    the size of the K and V caches together, streamed in one launch by rattn_read_probe
    (whole (page, KV head) blocks in a random order, non-temporal 16-byte loads, 1 KiB
    per 64-lane pass), rotated over enough copies that no pass hits in the caches."""
    import torch
    from decode_attention_verify_amd import binding
    elem = 1 if fp8 else 2
    block = sp.page_size * sp.head_dim * elem
    nblocks = 2 * case.k_cache.numel() * elem // block
    byts = nblocks * block
    ncopies = max(2, min(4, math.ceil(CACHE_EVICT_BYTES / byts) + 1))
    bufs = [torch.ones(byts, dtype=torch.uint8, device="cuda") for _ in range(ncopies)]
    g = torch.Generator(device="cuda").manual_seed(seed)
    order = torch.randperm(nblocks, generator=g, device="cuda").to(torch.int32)
    sink = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    vp = ctypes.c_void_p

    def rate(waves):
        def one(i):
            st = lib.rattn_read_probe(vp(bufs[i % ncopies].data_ptr()), nblocks, block,
                                      vp(order.data_ptr()), waves, vp(sink.data_ptr()),
                                      vp(stream.cuda_stream))
            if st != binding.RATTN_OK:
                raise binding.RattnError(st, "rattn_read_probe")
        for i in range(2):
            one(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps):
            one(i)
        e1.record()
        torch.cuda.synchronize()
        return byts / (e0.elapsed_time(e1) * 1e-3 / reps) / 1e9
    # 4 and 8 single-wave work-groups per CU (32 and 64 KiB in flight per CU at 4 KiB
    # blocks): either can be the faster on a given device; the ceiling is the better one
    by_waves = {w: rate(w) for w in (4 * num_cus, 8 * num_cus)}
    del bufs
    waves = max(by_waves, key=by_waves.get)
    best = by_waves[waves]
    return {"GBps": round(best, 1),
            "frac_of_peak": round(best / HBM_PEAK_GBPS, 4),
            "GBps_by_workgroups": {str(w): round(v, 1) for w, v in by_waves.items()},
            "bytes_per_pass": byts,
            "pattern": "%d blocks of %d B (the K and V caches' size) in a random order, "
                       "non-temporal 16-byte loads, 1 KiB per 64-lane pass, the better of %s "
                       "single-wave work-groups, one launch each (rattn_read_probe)"
                       % (nblocks, block, " and ".join(str(w) for w in by_waves))}


def parity_of(out_gpu, lse_gpu, ref_out, ref_lse):
    import numpy as np
    sel = ~np.isnan(ref_lse)
    if not sel.any():
        return None
    o = out_gpu.float().cpu().numpy().astype(np.float64)
    l = lse_gpu.cpu().numpy().astype(np.float64)
    osel = np.broadcast_to(sel[..., None], ref_out.shape)
    d = np.abs(o[osel] - ref_out[osel])
    rel = np.abs(l[sel] - ref_lse[sel]) / np.maximum(np.abs(ref_lse[sel]), 1.0)
    return {"rows_checked": int(sel.sum()), "max_abs": float(d.max()),
            "mean_abs": float(d.mean()), "lse_rel": float(rel.max())}


def bench_append(args, sp, case, prob):
    """Time rattn_append_kv: each sequence's n newest K and V rows written into the
    paged cache (quantised to E4M3 with per-row scales for the FP8 cache)."""
    import torch
    from decode_attention_verify_amd import accounting, binding
    fp8 = sp.kv_format == "fp8_e4m3"
    g = torch.Generator(device="cuda").manual_seed(args.seed + 1)
    shape = (sp.batch, sp.n_rows, sp.num_kv_heads, sp.head_dim)
    k_new = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
    v_new = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    byts = accounting.append_traffic(case.seq_lens.tolist(), n_rows=sp.n_rows,
                                     num_kv_heads=sp.num_kv_heads, head_dim=sp.head_dim,
                                     page_size=sp.page_size, kv_bytes_per_elem=1 if fp8 else 2)

    # one checked call through the binding, then the same arguments pre-marshalled, so
    # that the timed loop measures the library and not Python's argument checks
    binding.rattn_append_kv(prob, k_new, v_new, case.page_table, case.seq_lens, case.k_cache,
                            case.v_cache, case.k_scale, case.v_scale, flags)
    vp = ctypes.c_void_p
    p = lambda t: None if t is None else vp(t.data_ptr())   # noqa: E731
    argv = (ctypes.byref(prob), p(k_new), p(v_new), p(case.page_table), p(case.seq_lens),
            p(case.k_cache), p(case.v_cache), p(case.k_scale), p(case.v_scale), p(flags),
            vp(torch.cuda.current_stream().cuda_stream))
    fn = binding.load().rattn_append_kv

    def call():
        st = fn(*argv)
        if st != binding.RATTN_OK:
            raise binding.RattnError(st, "rattn_append_kv")
    settle_ms = settle(args.settle_ms)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # events on torch's current stream, the stream the binding launches on
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if int(flags.item()):
        raise RuntimeError("device flags %d on valid input" % int(flags.item()))
    us = (t1 - t0) * 1e6 / args.steps
    dev_us = e0.elapsed_time(e1) * 1e3 / args.steps
    print(json.dumps({
        "metric": "kv-cache append µs/call (n new tokens per sequence, K and V)",
        "value": round(us, 3), "unit": "us/call", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_ms": round(settle_ms, 1), "higher_is_better": False,
        "dtype": "bf16->" + sp.kv_format,
        "data": "synthetic",
        "config": {"workload": "append before: " + WORKLOADS[args.workload],
                   "name": args.workload, "batch": sp.batch, "n_new_tokens": sp.n_rows,
                   "kv_heads": sp.num_kv_heads, "page_size": sp.page_size},
        "device_us_per_call": round(dev_us, 3),
        "algorithmic_bytes": byts,
        "roofline": {"bound": "hbm", "kernel": "append_kv_kernel",
                     "achieved": round(byts / (dev_us * 1e-6) / 1e9, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(byts / (dev_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 5),
                     "traffic": None},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="full_100k", choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--splits", type=int, default=0, help="force the split count (0 = planner)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-stride", type=int, default=1,
                    help="in the kernel-timing pass, stamp every N-th step's kernels")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time the steps without the per-kernel HIP events (no roofline)")
    ap.add_argument("--op", default="decode", choices=("decode", "append"),
                    help="decode: the attention call (default); append: the KV-cache write "
                         "of each sequence's new tokens, on the same workload's shapes")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the streaming-read probe over the same K/V caches")
    ap.add_argument("--hot-cache", action="store_true",
                    help="after the timed steps, time as many on one input copy (a warm-cache "
                         "figure, reported beside the main one)")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="before the warm-up steps, keep the GPU busy this long with "
                         "scratch matrix products and copies (not the attention path, not "
                         "its inputs), so that the timed steps start at steady clocks")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this attention path runs on a single "
              "device and has no multi-GPU mode (got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_attention_verify_amd import accounting, binding, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(args.copy_probe, max(args.steps, 1))
        return

    lib = binding.load()              # raises if librattn.so is missing: no fallback
    sp = synth.spec(args.workload)
    say("workload", args.workload, "seed", args.seed)
    t = time.perf_counter()
    case = synth.make_case(sp, seed=args.seed, device="cuda", poison=False)
    torch.cuda.synchronize()
    say("inputs drawn in %.1fs" % (time.perf_counter() - t))
    fp8 = sp.kv_format == synth.KV_FP8
    rows = None
    if sp.rows_seed is not None:                 # rows per sequence of their own
        rows = synth.draw_rows_per_seq(sp.batch, sp.n_rows, seed=sp.rows_seed,
                                       allow_zero=False)
        q_packed, cu_rows = synth.varlen_rows(case, rows)
        case = dataclasses.replace(case, q=q_packed)
        say("rows per sequence", rows)
    tr = accounting.traffic(case.seq_lens.tolist(), n_rows=sp.n_rows,
                            num_q_heads=sp.num_q_heads, num_kv_heads=sp.num_kv_heads,
                            head_dim=sp.head_dim, window=sp.window, dmax=sp.dmax,
                            page_size=sp.page_size, kv_bytes_per_elem=1 if fp8 else 2,
                            rows_per_seq=rows)

    prob = binding.problem_from_case(case, args.splits)
    if args.op == "append" and rows is not None:
        raise SystemExit("--op append takes a workload with the same rows in every sequence")
    if args.op == "append":
        bench_append(args, sp, case, prob)
        return
    t = time.perf_counter()
    for _ in range(PLAN_REPS):
        binding.rattn_free(binding.rattn_plan(prob))
    plan_us = (time.perf_counter() - t) / PLAN_REPS * 1e6
    plan = binding.Plan(prob)
    info = plan.info.as_dict()
    say("plan", info)

    # copies of the streamed inputs, so consecutive steps never hit in the caches
    per_copy = sum(t.numel() * t.element_size() for t in
                   (case.q, case.k_cache, case.v_cache, case.bias) +
                   ((case.k_scale, case.v_scale) if fp8 else ()))
    ncopies = max(1, min(8, math.ceil(CACHE_EVICT_BYTES / per_copy)))
    copies = [case]
    for _ in range(ncopies - 1):
        copies.append(dataclasses.replace(
            case, q=case.q.clone(), k_cache=case.k_cache.clone(),
            v_cache=case.v_cache.clone(), bias=case.bias.clone(),
            k_scale=None if case.k_scale is None else case.k_scale.clone(),
            v_scale=None if case.v_scale is None else case.v_scale.clone()))
    out_rows = (sp.batch, sp.n_rows) if rows is None else (case.q.shape[0],)
    out = torch.empty(out_rows + (sp.num_q_heads, sp.head_dim), dtype=torch.bfloat16,
                      device="cuda")
    lse = torch.empty(out_rows + (sp.num_q_heads,), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    vp = ctypes.c_void_p
    p = lambda t: None if t is None else vp(t.data_ptr())   # noqa: E731
    if rows is None:
        binding.check_shapes(prob, case.q, case.k_cache, case.v_cache, case.k_scale,
                             case.v_scale, case.page_table, case.seq_lens, case.bias, out, lse)
        decode = lib.rattn_decode

        def argv(c):
            return (plan.handle, p(c.q), p(c.k_cache), p(c.v_cache), p(c.k_scale),
                    p(c.v_scale), p(c.page_table), p(c.seq_lens), p(c.bias), p(out), p(lse),
                    vp(stream.cuda_stream))
    else:
        # one checked call through the binding; the timed calls reuse its arguments
        plan.decode_varlen(case.q, case.k_cache, case.v_cache, case.k_scale, case.v_scale,
                           case.page_table, case.seq_lens, cu_rows, case.bias, out, lse)
        decode = lib.rattn_decode_varlen

        def argv(c):
            return (plan.handle, p(c.q), p(c.k_cache), p(c.v_cache), p(c.k_scale),
                    p(c.v_scale), p(c.page_table), p(c.seq_lens), p(cu_rows),
                    ctypes.c_int32(int(c.q.shape[0])), p(c.bias), p(out), p(lse),
                    vp(stream.cuda_stream))
    calls = [argv(c) for c in copies]

    def step(i):
        st = decode(*calls[i % ncopies])
        if st != binding.RATTN_OK:
            raise binding.RattnError(st, "decode")

    settle_ms = settle(args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    say("warmup done (%.0f ms of scratch copies, then %d steps, %d input copies, %.0f MB "
        "each)" % (settle_ms, args.warmup, ncopies, per_copy / 1e6))

    prefill_plan = info["kernel"] == binding.RATTN_KERNEL_PREFILL
    K = args.steps
    # pass 1, the figure: K steps back to back between two device synchronisations,
    # launched as a caller would launch them (no instrumentation)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # pass 2, the kernels: the same K steps, every stride-th launched with events that
    # the runtime stamps with each kernel's own start and end (stamping adds launch
    # overhead, which is why this pass is not the figure)
    stride = max(1, args.event_stride)
    nrec = (K + stride - 1) // stride
    if args.no_kernel_events:
        split_ms, comb_ms = [float("nan")], [float("nan")]
    else:
        binding.rattn_profile_begin(plan.handle, nrec, stride)
        for i in range(K):
            step(i)
        split_ms, comb_ms = binding.rattn_profile_end(plan.handle, nrec)
    # pass 3, single steps: the same K steps, each between a pair of events on the launch
    # stream (the events add their own small gaps)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    for i in range(K):
        evs[i].record()
        step(i)
    evs[K].record()
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(K))

    def pct(v, f):
        return round(v[min(len(v) - 1, int(f * len(v)))], 3)
    step_stats = {"mean": round(sum(per_step) / K, 3), "median": pct(per_step, 0.5),
                  "p10": pct(per_step, 0.1), "p90": pct(per_step, 0.9), "samples": K,
                  "how": "a third pass of the same steps, each between two events on "
                         "the launch stream"}
    hot_us = None
    if args.hot_cache:
        # secondary: the same steps on one input copy, whose K/V partly stay in the caches
        torch.cuda.synchronize()
        th = time.perf_counter()
        for i in range(K):
            step(0)
        torch.cuda.synchronize()
        hot_us = round((time.perf_counter() - th) * 1e6 / K, 3)
    probe = None
    if not args.no_read_probe and not prefill_plan:
        probe = read_probe(lib, case, sp, fp8, info["num_cus"])
        say("read probe: %.0f GB/s" % probe["GBps"])
    flags = plan.debug_flags()
    if flags:
        raise RuntimeError("device flags %d on valid input" % flags)
    ms_per_step = (t1 - t0) * 1e3 / K
    us = ms_per_step * 1e3
    say("timed %d steps: %.2f us/step" % (K, us))

    split_mean_s = sum(split_ms) / len(split_ms) * 1e-3
    srt = sorted(split_ms)
    split_bytes = tr.kv + tr.scales + tr.bias + tr.q + tr.page_table + tr.seq_lens
    if info["num_splits"] == 1:
        split_bytes += tr.out + tr.lse
    achieved = split_bytes / split_mean_s / 1e9
    prefill = info["kernel"] == binding.RATTN_KERNEL_PREFILL
    digest = kernel_digest()
    traffic = read_traffic(args.workload, digest)
    result = {
        "metric": METRIC,
        "value": round(us, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_ms": round(settle_ms, 1),
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic: bf16 matrix operands with fp32 accumulation and softmax (an
        # E4M3 cache is decoded exactly to bf16; config.kv_cache names the storage)
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOADS[args.workload],
            "name": args.workload,
            "batch": sp.batch,
            "n_query_rows": sp.n_rows if rows is None else rows,
            "q_heads": sp.num_q_heads,
            "kv_heads": sp.num_kv_heads,
            "head_dim": sp.head_dim,
            "seq_lens": (case.seq_lens.tolist() if sp.batch <= 16
                         else "%d sequences, sum %d" % (sp.batch, int(case.seq_lens.sum()))),
            "window": sp.window,
            "dmax": sp.dmax,
            "page_size": sp.page_size,
            "kv_cache": sp.kv_format,
            "num_splits": info["num_splits"],
            "keys_per_split": info["keys_per_split"],
            "parallelism": "single GPU",
            "seed": args.seed,
        },
        "algorithmic_bytes": tr.total,
        "hbm_GBps": round(tr.total / (us * 1e-6) / 1e9, 1),
        "TFLOPs": round(tr.flops / (us * 1e-6) / 1e12, 2),
        "hbm_frac_of_peak": round(tr.total / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "step_us": step_stats,
        "kernels_us": {
            "split_kv_mean": round(split_mean_s * 1e6, 3),
            "split_kv_median": round(srt[len(srt) // 2] * 1e3, 3),
            "split_kv_p10": round(srt[len(srt) // 10] * 1e3, 3),
            "split_kv_p90": round(srt[(len(srt) * 9) // 10] * 1e3, 3),
            "combine_mean": round(sum(comb_ms) / len(comb_ms) * 1e3, 3),
            "samples": len(split_ms),
            "event_stride": stride,
        },
        "plan_host_us": round(plan_us, 1),
        "hot_cache_us_per_step": hot_us,
        "roofline": ({
            "bound": "hbm",
            "kernel": "split_kv_kernel",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": split_bytes,
            "kernel_digest": digest,
        } if not prefill else {
            # a chunk of thousands of rows is a dense contraction: priced against the
            # bf16 matrix peak, 4 D flops per (row, query head, visible key)
            "bound": "mfma",
            "kernel": "prefill_e4m3_kernel" if fp8 else "prefill_kernel",
            "achieved": round(tr.flops / split_mean_s / 1e12, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tr.flops / split_mean_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
            "algorithmic_flops_per_launch": tr.flops,
        }),
        "input_copies": ncopies,
        "read_probe": probe,
    }

    if not args.no_cpu_baseline:
        say("cpu baseline: oracle on the host cores (budget %.0fs)" % args.cpu_budget)
        case_cpu = case.to("cpu")
        if prefill:
            cb, ref_out, ref_lse = cpu_baseline_rows(case_cpu, tr, args.cpu_budget)
        else:
            cb, ref_out, ref_lse = cpu_baseline(case_cpu, tr, args.cpu_budget, rows,
                                                None if rows is None else case_cpu.q,
                                                None if rows is None else cu_rows.cpu())
        result["cpu_baseline"] = cb
        # the last step's output against the oracle on the units it computed
        result["parity_vs_oracle"] = parity_of(out, lse, ref_out, ref_lse)
    else:
        result["cpu_baseline"] = None
    plan.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
