#!/usr/bin/env python3
"""Benchmark: grouped-query attention forward on one MI355X.

One step = one causal prefill forward of the Llama-3-8B-shaped workload (B=1, T=4096, 32 query /
8 key-value heads, d=128, bf16), inputs already resident in HBM. Prints ONE JSON line with the
prefill throughput (TFLOP/s of algorithmic work: 4*d flops per unmasked (query, key, head)
triple), its fraction of the bf16 matrix-core peak, the batched-decode KV-stream bandwidth
(B=64, 8192-entry cache) as a secondary figure, and the fp64 CPU oracle timed on a bounded
sample of the same prefill workload.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-decode]
                  [--only prefill|decode|mqa|varlen] [--all]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_HBM_GBS = 8000.0       # HBM3E
CSRC = os.path.join(ROOT, "grouped_query_softmax_amd", "csrc")
# HBM bytes per launch from the FETCH_SIZE / WRITE_SIZE counters (calibrated against a plain
# copy), valid only for the kernel sources they were taken on (checked by hash)
TRAFFIC = {
    "prefill": (os.path.join(ROOT, "profiles", "prefill_bf16_llama3_8b_T4096_traffic.json"),
                ("prefill_bf16.hip", "common.hpp")),
    "decode": (os.path.join(ROOT, "profiles", "decode_bf16_B64_kv8192_traffic.json"),
               ("decode.hip", "common.hpp")),
    "gva": (os.path.join(ROOT, "profiles", "gva_prefill_B2_T4096_H16_HV32_d64_traffic.json"),
            ("prefill_bf16.hip", "common.hpp")),
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def visible_pairs(Tq, Tkv, causal):
    """Unmasked (query, key) pairs of one head of one item (bottom-right causal alignment)."""
    if not causal:
        return Tq * Tkv
    off = Tkv - Tq
    return Tq * (off + 1) + Tq * (Tq - 1) // 2


def visible_pairs_window(T, window, n_sink):
    """Unmasked (query, key) pairs of one head of a square causal item with a sliding window of
    `window` keys plus `n_sink` sink keys below it."""
    pairs = 0
    for t in range(T):
        below = t + 1 - window  # keys 0 .. below-1 lie under the window
        pairs += min(t + 1, window) + (min(n_sink, below) if below > 0 else 0)
    return pairs


def prefill_flops(w):
    if w.window > 0:
        assert w.seqlens is None and w.Tq == w.Tkv
        pairs = w.B * visible_pairs_window(w.Tq, w.window, w.n_sink)
    elif w.seqlens is not None:
        pairs = sum(visible_pairs(n, n, w.causal) for n in w.seqlens)
    else:
        pairs = w.B * visible_pairs(w.Tq, w.Tkv, w.causal)
    return 4 * w.d * w.Hq * pairs


def kernel_source_sha(which="prefill"):
    h = hashlib.sha256()
    for name in TRAFFIC[which][1]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def device_inputs(w, torch, seed_base):
    """Seeded synthetic N(0,1) bf16 inputs drawn on the device (same shapes as the parity
    workloads; the parity tests draw on the host with the same recipe)."""
    g = torch.Generator(device="cuda")
    tot = sum(w.seqlens) if w.seqlens else None
    Tq = tot if tot else w.Tq
    Tkv = tot if tot else w.Tkv
    g.manual_seed(seed_base)
    q = torch.randn(w.B, Tq, w.Hq, w.d, generator=g, device="cuda", dtype=torch.float32)
    if w.peaked_frac > 0:
        nrows = q.numel() // w.d
        sel = torch.randperm(nrows, generator=g, device="cuda")[:int(round(w.peaked_frac * nrows))]
        q.view(nrows, w.d)[sel] *= w.peaked_scale
    q = q.to(torch.bfloat16)
    k = torch.randn(w.B, Tkv, w.Hkv, w.d, generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn(w.B, Tkv, w.Hkv, w.d, generator=g, device="cuda").to(torch.bfloat16)
    cu = None
    if w.seqlens:
        cu = torch.tensor(w.cu_seqlens, dtype=torch.int32, device="cuda")
    return q, k, v, cu


def time_launches(fn, steps, warmup, torch):
    """Times `steps` launches on the stream the kernels are launched on (torch's current stream,
    which the binding passes to the library): after `warmup` untimed launches, exactly `steps`
    back-to-back launches between two synchronizations, bracketed by one pair of HIP events on
    that stream. Returns (average ms per launch, wall-clock s of the timed region). Back to back
    the chip runs at its sustained (lower) clock; a kernel trace of the same command averages
    the same duration per launch."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def bench_prefill(gqa, w, steps, warmup, torch, seed, rope=False, qk_norm=False,
                  prepared=False):
    """rope: turn q and k inside the kernel with (cos, sin) tables (rotary embedding); qk_norm:
    RMSNorm of q and k (weights 1 + N(0, 0.1^2), eps 1e-6) before the rotation; prepared: each
    step runs gqa_prepare_keys (keys normalised / turned once) and then the attention with
    keys_prepared, both timed."""
    q, k, v, cu = device_inputs(w, torch, seed)
    out = torch.empty_like(q)
    msl = max(w.seqlens) if w.seqlens else None
    tables = None
    if rope:
        import workloads
        tables = tuple(torch.from_numpy(t).cuda() for t in workloads.rope_tables(w.Tkv, w.d))
    norm = None
    if qk_norm:
        g = torch.Generator(device="cuda")
        g.manual_seed(seed + 11)
        wq = 1 + 0.1 * torch.randn(w.d, generator=g, device="cuda")
        wk = 1 + 0.1 * torch.randn(w.d, generator=g, device="cuda")
        norm = (wq, wk, 1e-6)

    kbuf = torch.empty_like(k) if prepared else None

    def step():
        if prepared:
            gqa.gqa_prepare_keys(k, rope=tables, qk_norm=norm, out=kbuf)
            gqa.gqa_attn_prefill_ex(q, kbuf, v, causal=w.causal, rope=tables, qk_norm=norm,
                                    keys_prepared=True, out=out)
        elif tables is not None or norm is not None:
            gqa.gqa_attn_prefill_ex(q, k, v, causal=w.causal, window=w.window, n_sink=w.n_sink,
                                    rope=tables, qk_norm=norm, out=out)
        elif w.window > 0:
            gqa.gqa_attn_prefill_window(q, k, v, window=w.window, n_sink=w.n_sink, out=out)
        else:
            gqa.gqa_attn_prefill(q, k, v, causal=w.causal, cu_seqlens=cu, max_seqlen=msl, out=out)

    avg, wall = time_launches(step, steps, warmup, torch)
    flops = prefill_flops(w)
    res = {"workload": w.name, "flops_per_launch": flops, "avg_ms": avg,
           "tflops": flops / (avg * 1e-3) / 1e12, "wall_s": wall}
    return res, (q, k, v, cu)


def bench_backward(gqa, w, steps, warmup, torch, seed):
    """Backward of the causal prefill (dq, dk, dv): algorithmic work is 10*d flops per unmasked
    (query, key, head) triple (recomputed scores, dP, dV, dK, dQ), 2.5x the forward's."""
    q, k, v, _ = device_inputs(w, torch, seed)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 7)
    dout = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    out = gqa.gqa_attn_prefill_ex(q, k, v, causal=w.causal, lse=lse)
    ws = torch.empty(gqa.raw_library().gqa_attn_backward_workspace_bytes(w.B, w.Tq, w.Hq),
                     dtype=torch.uint8, device="cuda")

    def step():
        gqa.gqa_attn_backward(q, k, v, out, dout, lse, causal=w.causal, workspace=ws)

    avg, wall = time_launches(step, steps, warmup, torch)
    flops = prefill_flops(w) * 10 // 4
    return {"workload": w.name + "+backward", "flops_per_launch": flops, "avg_ms": avg,
            "tflops": flops / (avg * 1e-3) / 1e12,
            "frac_mfma": flops / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "wall_s": wall}


def bench_gva(gqa, w, steps, warmup, torch, seed):
    """Grouped value attention prefill (H = w.Hkv query/key heads, HV = w.Hq value heads):
    algorithmic work per unmasked (query, key, query/key head) pair is 2*d for the score and
    2*d per value head for the weighted sum, 2*d*(1 + G)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    H, HV = w.Hkv, w.Hq
    q = torch.randn(w.B, w.Tq, H, w.d, generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn(w.B, w.Tkv, H, w.d, generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn(w.B, w.Tkv, HV, w.d, generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty(w.B, w.Tq, HV, w.d, dtype=torch.bfloat16, device="cuda")

    def step():
        gqa.gqa_attn_prefill_gva(q, k, v, causal=w.causal, out=out)

    avg, wall = time_launches(step, steps, warmup, torch)
    flops = 2 * w.d * (H + HV) * w.B * visible_pairs(w.Tq, w.Tkv, w.causal)
    return {"workload": w.name, "flops_per_launch": flops, "avg_ms": avg,
            "tflops": flops / (avg * 1e-3) / 1e12,
            "frac_mfma": flops / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "wall_s": wall}


def bench_decode(gqa, w, steps, warmup, torch, seed):
    """Alternates two distinct caches (4 GiB together) so no run rides the previous one's
    last-level cache."""
    sets = []
    for i in range(2):
        q, k, v, _ = device_inputs(w, torch, seed + 10 * i)
        sets.append((q, k, v))
    ws = torch.empty(gqa.gqa_attn_decode_workspace_bytes(w.B, w.Tkv, w.Hq, w.d),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(sets[0][0])
    lens = None
    if w.cache_lens is not None:
        lens = torch.tensor(w.cache_lens, dtype=torch.int32, device="cuda")
    it = [0]

    def step():
        q, k, v = sets[it[0] & 1]
        it[0] += 1
        if lens is not None:
            gqa.gqa_attn_decode_ragged(q, k, v, cache_lens=lens, workspace=ws, out=out)
        else:
            gqa.gqa_attn_decode(q, k, v, workspace=ws, out=out)

    avg, wall = time_launches(step, steps, warmup, torch)
    entries = sum(w.cache_lens) if w.cache_lens is not None else w.B * w.Tkv
    kv_bytes = 2 * entries * w.Hkv * w.d * 2
    qo_bytes = 2 * w.B * w.Hq * w.d * 2
    gbs = (kv_bytes + qo_bytes) / (avg * 1e-3) / 1e9
    return {"workload": w.name, "bytes_per_launch": kv_bytes + qo_bytes, "avg_ms": avg,
            "gbs": gbs, "frac_hbm": gbs / PEAK_HBM_GBS, "wall_s": wall,
            "traffic": traffic_for("decode") if w.cache_lens is None else None}


FOLD_SHAPE = (8, 4096, 32, 128, 8)  # B, T, H, d, g: a 32-head K (or V) folded to 8 heads


def bench_fold(gqa, steps, warmup, torch):
    """gqa_fold_kv on a multi-head key tensor [B, T, H, d] folded to g heads (the step that
    turns a multi-head checkpoint or cache into a grouped one): reads B*T*H*d and writes B*T*g*d
    bf16 values once each; HBM-bound."""
    B, T, H, d, g = FOLD_SHAPE
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9000)
    src = torch.randn(B, T, H, d, generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty(B, T, g, d, dtype=torch.bfloat16, device="cuda")
    avg, wall = time_launches(lambda: gqa.gqa_fold_kv(src, g, out=out), steps, warmup, torch)
    nbytes = (B * T * H * d + B * T * g * d) * 2
    gbs = nbytes / (avg * 1e-3) / 1e9
    return {"metric": "fold_kv GB/s (read + write, % HBM peak)", "value": gbs, "unit": "GB/s",
            "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": avg,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) on device)",
            "config": {"workload": f"fold_B{B}_T{T}_H{H}_g{g}_d{d}", "B": B, "T": T, "H": H,
                       "g": g, "d": d},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "traffic": None,
                         "kernel": "fold_kernel<BF16>", "bytes_per_launch": nbytes,
                         "avg_launch_ms": avg},
            "cpu_baseline": None, "wall_s": wall}


COPY_BYTES = 1 << 30


def bench_copy(steps, warmup, torch):
    """A plain device-to-device copy of COPY_BYTES: it reads and writes exactly COPY_BYTES each,
    so the HBM byte counters it reports calibrate those of the attention kernels."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    avg, wall = time_launches(lambda: dst.copy_(src), steps, warmup, torch)
    gbs = 2 * COPY_BYTES / (avg * 1e-3) / 1e9
    return {"metric": "device copy GB/s (read + write)", "value": gbs, "unit": "GB/s",
            "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": avg,
            "higher_is_better": True, "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
            "config": {"workload": "copy_1GiB"}}


def cpu_baseline(w, tensors, torch, target_s=15.0):
    """fp64 oracle on a bounded sample of the prefill workload: the first `ng` key/value heads
    with their G query heads each (the same grouping; every query position, every key)."""
    import numpy as np

    import oracle
    import workloads
    orc = oracle.default()
    q, k, v, _ = tensors
    G = w.Hq // w.Hkv

    def run(ng):
        qs = workloads.bf16_bits(q[:, :, :G * ng].contiguous().cpu())
        ks = workloads.bf16_bits(k[:, :, :ng].contiguous().cpu())
        vs = workloads.bf16_bits(v[:, :, :ng].contiguous().cpu())
        t0 = time.perf_counter()
        orc.attention(qs, ks, vs, causal=w.causal)
        return time.perf_counter() - t0

    # calibrate on a small sample, then size the timed sample for ~target_s seconds
    t1 = run(1)
    ng = max(1, min(w.Hkv, int(target_s / max(t1, 1e-3))))
    t = t1 if ng == 1 else run(ng)
    flops = 4 * w.d * (G * ng) * w.B * visible_pairs(w.Tq, w.Tkv, w.causal)
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": orc.num_threads(),
            "kind": "oracle",
            "sample": f"{w.name}: key/value heads 0..{ng - 1} with their {G * ng} query heads "
                      f"(of {w.Hq}), all {w.Tq} positions, causal; {flops / 1e9:.1f} GFLOP in "
                      f"{t:.1f} s, fp64"}


def traffic_for(which):
    """Calibrated HBM bytes per launch, or None when no counters exist for the current source."""
    path = TRAFFIC[which][0]
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_sha(which):
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "mqa", "varlen", "window",
                                       "ragged", "rope", "qknorm", "backward", "gva",
                                       "fold", "copy"],
                    default=None,
                    help="time a single workload (for profiling); still prints one JSON line. "
                         "'copy' times a plain 1 GiB device copy, the calibration kernel for "
                         "the HBM byte counters; 'fold' times gqa_fold_kv")
    ap.add_argument("--all", action="store_true", help="also time the MQA and varlen prefills")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (a multi-GPU "
              f"run would shard the key/value heads, one process per GPU)", file=sys.stderr)
        sys.exit(2)

    import torch

    import grouped_query_softmax_amd as gqa
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.only == "copy":
        print(json.dumps(bench_copy(args.steps, args.warmup, torch)), flush=True)
        return
    if args.only == "fold":
        res = bench_fold(gqa, args.steps, args.warmup, torch)
        log(f"fold: {res['ms_per_step'] * 1e3:.1f} us, {res['value']:.0f} GB/s")
        print(json.dumps(res), flush=True)
        return

    w = workloads.LLAMA_PREFILL
    extra = {}
    pre = None
    tensors = None
    if args.only in (None, "prefill"):
        log(f"prefill {w.name}: {args.warmup} warmup + {args.steps} timed launches")
        pre, tensors = bench_prefill(gqa, w, args.steps, args.warmup, torch, 2000)
        log(f"prefill: {pre['avg_ms'] * 1e3:.1f} us avg, {pre['tflops']:.1f} TFLOP/s")
    if args.only == "mqa" or args.all:
        m, _ = bench_prefill(gqa, workloads.MQA_PREFILL, args.steps, args.warmup, torch, 4000)
        m["frac_mfma"] = m["tflops"] / PEAK_BF16_TFLOPS
        extra["mqa_prefill"] = m
        log(f"mqa: {m['avg_ms'] * 1e3:.1f} us, {m['tflops']:.1f} TFLOP/s")
    if args.only == "varlen" or args.all:
        vl, _ = bench_prefill(gqa, workloads.VARLEN_PREFILL, max(5, args.steps // 5),
                              args.warmup, torch, 5000)
        vl["frac_mfma"] = vl["tflops"] / PEAK_BF16_TFLOPS
        extra["varlen_prefill"] = vl
        log(f"varlen: {vl['avg_ms']:.3f} ms, {vl['tflops']:.1f} TFLOP/s")
    if args.only == "window" or args.all:
        wp, _ = bench_prefill(gqa, workloads.WINDOW_PREFILL, args.steps, args.warmup, torch, 6000)
        wp["frac_mfma"] = wp["tflops"] / PEAK_BF16_TFLOPS
        extra["window_prefill"] = wp
        log(f"window prefill: {wp['avg_ms'] * 1e3:.1f} us, {wp['tflops']:.1f} TFLOP/s")
    if args.only == "rope" or args.all:
        rp, _ = bench_prefill(gqa, workloads.LLAMA_PREFILL, args.steps, args.warmup, torch, 2000,
                              rope=True)
        rp["frac_mfma"] = rp["tflops"] / PEAK_BF16_TFLOPS
        rp["workload"] = workloads.LLAMA_PREFILL.name + "+rope"
        extra["rope_prefill"] = rp
        log(f"rope prefill: {rp['avg_ms'] * 1e3:.1f} us, {rp['tflops']:.1f} TFLOP/s")
        pp, _ = bench_prefill(gqa, workloads.LLAMA_PREFILL, args.steps, args.warmup, torch, 2000,
                              rope=True, prepared=True)
        pp["frac_mfma"] = pp["tflops"] / PEAK_BF16_TFLOPS
        pp["workload"] = workloads.LLAMA_PREFILL.name + "+rope, keys prepared"
        extra["rope_prefill_keys_prepared"] = pp
        log(f"rope prefill, keys prepared: {pp['avg_ms'] * 1e3:.1f} us, "
            f"{pp['tflops']:.1f} TFLOP/s")
    if args.only == "qknorm" or args.all:
        qn, _ = bench_prefill(gqa, workloads.LLAMA_PREFILL, args.steps, args.warmup, torch, 2000,
                              rope=True, qk_norm=True)
        qn["frac_mfma"] = qn["tflops"] / PEAK_BF16_TFLOPS
        qn["workload"] = workloads.LLAMA_PREFILL.name + "+qknorm+rope"
        extra["qknorm_rope_prefill"] = qn
        log(f"qk-norm + rope prefill: {qn['avg_ms'] * 1e3:.1f} us, {qn['tflops']:.1f} TFLOP/s")
        qp, _ = bench_prefill(gqa, workloads.LLAMA_PREFILL, args.steps, args.warmup, torch, 2000,
                              rope=True, qk_norm=True, prepared=True)
        qp["frac_mfma"] = qp["tflops"] / PEAK_BF16_TFLOPS
        qp["workload"] = workloads.LLAMA_PREFILL.name + "+qknorm+rope, keys prepared"
        extra["qknorm_rope_prefill_keys_prepared"] = qp
        log(f"qk-norm + rope prefill, keys prepared: {qp['avg_ms'] * 1e3:.1f} us, "
            f"{qp['tflops']:.1f} TFLOP/s")
    if args.only == "backward" or args.all:
        bw = bench_backward(gqa, workloads.LLAMA_PREFILL, args.steps, args.warmup, torch, 2000)
        extra["backward"] = bw
        log(f"backward: {bw['avg_ms'] * 1e3:.1f} us, {bw['tflops']:.1f} TFLOP/s")
    if args.only == "gva" or args.all:
        gv = bench_gva(gqa, workloads.GVA_PREFILL, args.steps, args.warmup, torch, 8000)
        extra["gva_prefill"] = gv
        log(f"gva prefill: {gv['avg_ms'] * 1e3:.1f} us, {gv['tflops']:.1f} TFLOP/s")
    if args.only == "ragged" or args.all:
        rd = bench_decode(gqa, workloads.RAGGED_DECODE, args.steps, args.warmup, torch, 7000)
        extra["ragged_decode"] = rd
        log(f"ragged decode: {rd['avg_ms'] * 1e3:.1f} us, {rd['gbs']:.0f} GB/s")
    if args.only == "decode" or (args.only is None and not args.no_decode):
        dec = bench_decode(gqa, workloads.DECODE, args.steps, args.warmup, torch, 3000)
        extra["decode"] = dec
        log(f"decode: {dec['avg_ms'] * 1e3:.1f} us, {dec['gbs']:.0f} GB/s")
    sha = kernel_source_sha("prefill")
    metric = "GQA prefill TFLOPS (% MFMA peak); decode KV GB/s (% HBM peak)"
    if pre is None and args.only in ("mqa", "varlen", "window", "rope", "qknorm", "backward",
                                     "gva"):
        key, w = {"gva": ("gva_prefill", workloads.GVA_PREFILL),
                  "qknorm": ("qknorm_rope_prefill", workloads.LLAMA_PREFILL),
                  "mqa": ("mqa_prefill", workloads.MQA_PREFILL),
                  "varlen": ("varlen_prefill", workloads.VARLEN_PREFILL),
                  "window": ("window_prefill", workloads.WINDOW_PREFILL),
                  "rope": ("rope_prefill", workloads.LLAMA_PREFILL),
                  "backward": ("backward", workloads.LLAMA_PREFILL)}[args.only]
        pre = extra.pop(key)
    if pre is not None:
        value, unit = pre["tflops"], "TFLOP/s"
        ms_per_step = pre["avg_ms"]
        traffic = None
        if args.only in (None, "prefill"):
            traffic = traffic_for("prefill")
        elif args.only == "gva":
            traffic = traffic_for("gva")
        roofline = {"bound": "mfma", "achieved": pre["tflops"], "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": pre["tflops"] / PEAK_BF16_TFLOPS,
                    "traffic": traffic,
                    "kernel": {"backward": "bwd_rowdot + bwd_dkdv_kernel<128> + bwd_dq_kernel<128>",
                               # <DQ, DV, ROPE, NORM, KPROC>: the fused variants process
                               # the keys in the kernel
                               "rope": "prefill_pp_kernel<128, 128, true, false, true>",
                               "qknorm": "prefill_pp_kernel<128, 128, true, true, true>",
                               "gva": "prefill_pp_kernel<64, 128, false, false, false>"}.get(
                                   args.only, "prefill_pp_kernel<128, 128, false, false, false>"),
                    "flops_per_launch": pre["flops_per_launch"],
                    "avg_launch_ms": pre["avg_ms"], "kernel_source_sha": sha}
        config = {"workload": w.name, "B": w.B, "T": w.Tq, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
                  "causal": w.causal, "global_batch": w.B, "seq_len": w.Tq,
                  "parallelism": "single-gpu"}
        if w.seqlens:
            config["seqlens"] = list(w.seqlens)
        if w.window > 0:
            config["window"], config["n_sink"] = w.window, w.n_sink
        if args.only == "gva":
            config.update({"H": w.Hkv, "HV": w.Hq})
            del config["Hq"], config["Hkv"]
    else:
        dw = workloads.RAGGED_DECODE if args.only == "ragged" else workloads.DECODE
        dec = extra.pop("ragged_decode" if args.only == "ragged" else "decode")
        value, unit = dec["gbs"], "GB/s"
        ms_per_step = dec["avg_ms"]
        roofline = {"bound": "hbm", "achieved": dec["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": dec["frac_hbm"], "traffic": dec["traffic"],
                    "kernel": "decode_split_kernel<128>", "bytes_per_launch":
                    dec["bytes_per_launch"], "avg_launch_ms": dec["avg_ms"],
                    "kernel_source_sha": kernel_source_sha("decode")}
        config = {"workload": dw.name, "B": dw.B, "Tkv": dw.Tkv, "Hq": dw.Hq, "Hkv": dw.Hkv,
                  "d": dw.d, "parallelism": "single-gpu"}
    line = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) on device)", "config": config,
            "roofline": roofline}
    if extra:
        line["secondary"] = extra
    if not args.no_cpu_baseline and tensors is not None:
        log("cpu baseline: fp64 oracle on a sample")
        line["cpu_baseline"] = cpu_baseline(w, tensors, torch)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
