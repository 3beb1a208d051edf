#!/usr/bin/env python3
"""Benchmark: grouped-query attention forward on one MI355X.

One step = one causal prefill forward of the packed long-context workload (four sequences of
16384 / 8192 / 4096 / 1024 tokens, 64 query / 8 key-value heads, d = 128, bf16), inputs already
resident in HBM: the largest configuration that fits one GPU. Prints ONE JSON line with its
throughput (TFLOP/s of algorithmic work: 4*d flops per unmasked (query, key, head) triple) and
fraction of the bf16 matrix-core peak, the other benchmark workloads as secondary legs with
their own roofline records (the 4096-token 32/8 prefill, the 8 x 2048-token multi-query prefill
with 5 % of the query rows scaled x30, and the 64-sequence decode against 8192-entry caches,
whose key/value stream is measured against the HBM peak), and the fp64 CPU oracle timed on a
bounded sample of the packed workload.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-secondary]
                  [--only varlen|prefill|decode|mqa|...] [--all]
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
    "varlen": (os.path.join(ROOT, "profiles", "prefill_bf16_varlen_16k_8k_4k_1k_traffic.json"),
               ("prefill_bf16.hip", "common.hpp")),
    "mqa": (os.path.join(ROOT, "profiles", "prefill_bf16_mqa_B8_T2048_traffic.json"),
            ("prefill_bf16.hip", "common.hpp")),
    "decode": (os.path.join(ROOT, "profiles", "decode_bf16_B64_kv8192_traffic.json"),
               ("decode.hip", "decode.hpp", "common.hpp")),
    "gva": (os.path.join(ROOT, "profiles", "gva_prefill_B2_T4096_H16_HV32_d64_traffic.json"),
            ("prefill_bf16.hip", "common.hpp")),
    "fold": (os.path.join(ROOT, "profiles", "fold_bf16_B8_T4096_H32_g8_d128_traffic.json"),
             ("fold.hip", "common.hpp")),
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


# kernel sources of legs that have no traffic record
SOURCES = {"backward": ("backward.hip", "backward.hpp", "common.hpp")}


def kernel_source_sha(which="prefill"):
    h = hashlib.sha256()
    for name in (TRAFFIC[which][1] if which in TRAFFIC else SOURCES[which]):
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


def time_launches(fn, steps, warmup, torch, per_launch=50):
    """Times `steps` launches on the stream the kernels are launched on (torch's current stream,
    which the binding passes to the library): after `warmup` untimed launches, exactly `steps`
    back-to-back launches between two synchronizations, bracketed by one pair of HIP events on
    that stream. Then, untimed for the average, `per_launch` more launches each bracketed by its
    own event pair, for the median and minimum launch time. Returns (average ms per launch of
    the timed region, wall-clock s of the timed region, median ms, min ms)."""
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
    avg = start.elapsed_time(end) / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(per_launch)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    each = sorted(a.elapsed_time(b) for a, b in evs)
    median = each[len(each) // 2] if each else avg
    return avg, wall, median, (each[0] if each else avg)


PER_LAUNCH = 50  # separately timed launches for the median and minimum (set by --median-launches)


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

    avg, wall, med, mn = time_launches(step, steps, warmup, torch, PER_LAUNCH)
    flops = prefill_flops(w)
    res = {"workload": w.name, "flops_per_launch": flops, "avg_ms": avg,
           "median_ms": med, "min_ms": mn,
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

    avg, wall, _, _ = time_launches(step, steps, warmup, torch, per_launch=0)
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

    avg, wall, _, _ = time_launches(step, steps, warmup, torch, per_launch=0)
    flops = 2 * w.d * (H + HV) * w.B * visible_pairs(w.Tq, w.Tkv, w.causal)
    return {"workload": w.name, "flops_per_launch": flops, "avg_ms": avg,
            "tflops": flops / (avg * 1e-3) / 1e12,
            "frac_mfma": flops / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "wall_s": wall}


def decode_entries(w):
    """Cache entries a decode step reads once, over all sequences: every entry of a plain cache,
    each sequence's first cache_lens[b] entries of a ragged one, and of a cache bounded to the
    window its sinks and window (the entries its query sees; the rest were written over)."""
    if w.window_cache:
        return sum(min(L, w.n_sink + w.window) for L in w.cache_lens)
    return sum(w.cache_lens) if w.cache_lens is not None else w.B * w.Tkv


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
        if w.window_cache:
            gqa.gqa_attn_decode_window_cache(q, k, v, lens, window=w.window, n_sink=w.n_sink,
                                             workspace=ws, out=out)
        elif lens is not None:
            gqa.gqa_attn_decode_ragged(q, k, v, cache_lens=lens, workspace=ws, out=out)
        else:
            gqa.gqa_attn_decode(q, k, v, workspace=ws, out=out)

    avg, wall, med, mn = time_launches(step, steps, warmup, torch, PER_LAUNCH)
    entries = decode_entries(w)
    kv_bytes = 2 * entries * w.Hkv * w.d * 2
    qo_bytes = 2 * w.B * w.Hq * w.d * 2
    gbs = (kv_bytes + qo_bytes) / (avg * 1e-3) / 1e9
    return {"workload": w.name, "bytes_per_launch": kv_bytes + qo_bytes, "avg_ms": avg,
            "median_ms": med, "min_ms": mn,
            "splits": gqa.gqa_attn_decode_workspace_bytes_hkv(w.B, w.Tkv, w.Hq, w.Hkv, w.d)
            // (w.B * w.Hq * (w.d + 2) * 4),
            "gbs": gbs, "frac_hbm": gbs / PEAK_HBM_GBS, "wall_s": wall,
            "traffic": traffic_for("decode", w.name)}


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
    avg, wall, _, _ = time_launches(lambda: gqa.gqa_fold_kv(src, g, out=out), steps, warmup,
                                    torch, per_launch=0)
    nbytes = (B * T * H * d + B * T * g * d) * 2
    gbs = nbytes / (avg * 1e-3) / 1e9
    return {"metric": "fold_kv GB/s (read + write, % HBM peak)", "value": gbs, "unit": "GB/s",
            "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": avg,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) on device)",
            "config": {"workload": f"fold_B{B}_T{T}_H{H}_g{g}_d{d}", "B": B, "T": T, "H": H,
                       "g": g, "d": d},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "traffic": traffic_for("fold"),
                         "kernel": "fold_kernel<BF16>", "bytes_per_launch": nbytes,
                         "avg_launch_ms": avg, "kernel_source_sha": kernel_source_sha("fold")},
            "cpu_baseline": None, "wall_s": wall}


COPY_BYTES = 1 << 30


def bench_copy(steps, warmup, torch):
    """A plain device-to-device copy of COPY_BYTES: it reads and writes exactly COPY_BYTES each,
    so the HBM byte counters it reports calibrate those of the attention kernels."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    avg, wall, _, _ = time_launches(lambda: dst.copy_(src), steps, warmup, torch, per_launch=0)
    gbs = 2 * COPY_BYTES / (avg * 1e-3) / 1e9
    return {"metric": "device copy GB/s (read + write)", "value": gbs, "unit": "GB/s",
            "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": avg,
            "higher_is_better": True, "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
            "config": {"workload": "copy_1GiB"}}


def cpu_baseline(w, tensors, torch, target_s=15.0):
    """fp64 oracle on a bounded sample of the prefill workload: the first `ng` key/value heads
    with their G query heads each (the same grouping; every query position, every key) of one
    item -- for a packed workload its 4096-token sequence, whose causal rows span the same
    lengths as the others' (oracle time, like the kernel's work, grows as T^2)."""
    import oracle
    import workloads
    orc = oracle.default()
    q, k, v, _ = tensors
    G = w.Hq // w.Hkv
    if w.seqlens:
        s = list(w.seqlens).index(4096) if 4096 in w.seqlens else 0
        a = int(w.cu_seqlens[s])
        T = w.seqlens[s]
        rows, what = slice(a, a + T), f"sequence {s} ({T} tokens)"
    else:
        T = w.Tq
        rows, what = slice(0, T), f"all {T} positions"

    def run(ng):
        qs = workloads.bf16_bits(q[:1, rows, :G * ng].contiguous().cpu())
        ks = workloads.bf16_bits(k[:1, rows, :ng].contiguous().cpu())
        vs = workloads.bf16_bits(v[:1, rows, :ng].contiguous().cpu())
        t0 = time.perf_counter()
        orc.attention(qs, ks, vs, causal=w.causal)
        return time.perf_counter() - t0

    # calibrate on a small sample, then size the timed sample for ~target_s seconds
    t1 = run(1)
    ng = max(1, min(w.Hkv, int(target_s / max(t1, 1e-3))))
    t = t1 if ng == 1 else run(ng)
    flops = 4 * w.d * (G * ng) * visible_pairs(T, T, w.causal)
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": orc.num_threads(),
            "kind": "oracle",
            "sample": f"{w.name}: {what} of item 0, key/value heads 0..{ng - 1} with their "
                      f"{G * ng} query heads (of {w.Hq}), causal; {flops / 1e9:.1f} GFLOP in "
                      f"{t:.1f} s, fp64"}


def traffic_for(which, workload=None):
    """Calibrated HBM bytes per launch, or None when no counters exist for the current source
    (or, when `workload` is given, for that workload)."""
    path = TRAFFIC[which][0]
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_sha(which):
        return None
    if workload is not None and rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


KERNEL_PLAIN = "prefill_pp_kernel<128, 128, false, false, false>"


def mfma_roofline(res, kernel, traffic_key=None, sha_key=None):
    """Roofline record of an MFMA-bound leg: algorithmic flops per launch over the measured
    average launch time, against the bf16 dense peak."""
    sha_key = sha_key or (traffic_key if traffic_key in TRAFFIC else "prefill")
    return {"bound": "mfma", "achieved": res["tflops"], "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": res["tflops"] / PEAK_BF16_TFLOPS,
            "traffic": traffic_for(traffic_key) if traffic_key else None, "kernel": kernel,
            "flops_per_launch": res["flops_per_launch"], "avg_launch_ms": res["avg_ms"],
            "median_launch_ms": res.get("median_ms"), "min_launch_ms": res.get("min_ms"),
            "kernel_source_sha": kernel_source_sha(sha_key)}


def hbm_roofline(res, kernel):
    return {"bound": "hbm", "achieved": res["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": res["frac_hbm"], "traffic": res.get("traffic"), "kernel": kernel,
            "bytes_per_launch": res["bytes_per_launch"], "avg_launch_ms": res["avg_ms"],
            "median_launch_ms": res.get("median_ms"), "min_launch_ms": res.get("min_ms"),
            "kernel_source_sha": kernel_source_sha("decode")}


def prefill_config(w):
    config = {"workload": w.name, "B": w.B, "T": w.Tq, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
              "causal": w.causal, "global_batch": w.B, "seq_len": w.Tq,
              "parallelism": "single-gpu"}
    if w.seqlens:
        config.update({"seqlens": list(w.seqlens), "global_batch": len(w.seqlens),
                       "seq_len": max(w.seqlens), "total_tokens": sum(w.seqlens)})
    if w.peaked_frac > 0:
        config.update({"peaked_rows": w.peaked_frac, "peaked_scale": w.peaked_scale})
    if w.window > 0:
        config["window"], config["n_sink"] = w.window, w.n_sink
    return config


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="time only the headline workload")
    ap.add_argument("--median-launches", type=int, default=50,
                    help="separately timed launches for the median and minimum (0: none)")
    ap.add_argument("--only", choices=["varlen", "prefill", "decode", "mqa", "window",
                                       "ragged", "longdecode", "windowcache", "rope", "qknorm",
                                       "backward",
                                       "gva", "fold", "copy"],
                    default=None,
                    help="time a single workload as the line's headline (for profiling); "
                         "'copy' times a plain 1 GiB device copy, the calibration kernel for the "
                         "HBM byte counters; 'fold' times gqa_fold_kv")
    ap.add_argument("--all", action="store_true",
                    help="also time the variant legs (window, ragged decode, long-context "
                         "decode, RoPE, QK-norm, backward, grouped values)")
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

    global PER_LAUNCH
    PER_LAUNCH = max(0, args.median_launches)
    S, Wu = args.steps, args.warmup
    headline = args.only or "varlen"
    legs = {}      # name -> (result, roofline, config)
    tensors = {}

    def run_prefill(name, w, seed, kernel=KERNEL_PLAIN, traffic_key=None, **kw):
        log(f"{name} {w.name}: {Wu} warmup + {S} timed launches")
        res, t = bench_prefill(gqa, w, S, Wu, torch, seed, **kw)
        tensors[name] = (w, t)
        log(f"{name}: {res['avg_ms'] * 1e3:.1f} us avg (median {res['median_ms'] * 1e3:.1f}, "
            f"min {res['min_ms'] * 1e3:.1f}), {res['tflops']:.1f} TFLOP/s")
        legs[name] = (res, mfma_roofline(res, kernel, traffic_key), prefill_config(w))

    def run_decode(name, w, seed):
        log(f"{name} {w.name}: {Wu} warmup + {S} timed launches")
        res = bench_decode(gqa, w, S, Wu, torch, seed)
        log(f"{name}: {res['avg_ms'] * 1e3:.1f} us, {res['gbs']:.0f} GB/s")
        cfg = {"workload": w.name, "B": w.B, "Tkv": w.Tkv, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
               "parallelism": "single-gpu"}
        if w.window_cache:
            cfg.update({"window": w.window, "n_sink": w.n_sink,
                        "entries_per_sequence": w.cache_lens[0]})
        elif w.cache_lens is not None:
            cfg["cache_lens"] = "uniform 1..Tkv (seeded)"
        kern = "decode_split_kernel<128, 1, {}>".format("true" if w.window_cache else "false")
        if res["splits"] > 1:
            kern += " + decode_combine_kernel<128>"
        legs[name] = (res, hbm_roofline(res, kern), cfg)

    plan = []
    if headline == "varlen" or not args.no_secondary and args.only is None:
        plan.append("varlen")
    if args.only is None and not args.no_secondary:
        plan += ["prefill", "mqa", "decode"]
    elif args.only not in (None, "varlen"):
        plan.append(args.only)
    if args.all:
        plan += [x for x in ("window", "ragged", "longdecode", "windowcache", "rope", "qknorm",
                             "backward", "gva") if x not in plan]

    for name in plan:
        if name == "varlen":
            run_prefill("varlen", workloads.VARLEN_PREFILL, 5000, traffic_key="varlen")
        elif name == "prefill":
            run_prefill("prefill", workloads.LLAMA_PREFILL, 2000, traffic_key="prefill")
        elif name == "mqa":
            run_prefill("mqa", workloads.MQA_PREFILL, 4000, traffic_key="mqa")
        elif name == "window":
            run_prefill("window", workloads.WINDOW_PREFILL, 6000)
        elif name == "rope":
            run_prefill("rope", workloads.LLAMA_PREFILL, 2000, rope=True,
                        kernel="prefill_pp_kernel<128, 128, true, false, true>")
            run_prefill("rope_keys_prepared", workloads.LLAMA_PREFILL, 2000, rope=True,
                        prepared=True,
                        kernel="prepare_keys_kernel + prefill_pp_kernel<128, 128, true, false, "
                               "false>")
        elif name == "qknorm":
            run_prefill("qknorm", workloads.LLAMA_PREFILL, 2000, rope=True, qk_norm=True,
                        kernel="prefill_pp_kernel<128, 128, true, true, true>")
            run_prefill("qknorm_keys_prepared", workloads.LLAMA_PREFILL, 2000, rope=True,
                        qk_norm=True, prepared=True,
                        kernel="prepare_keys_kernel + prefill_pp_kernel<128, 128, true, true, "
                               "false>")
        elif name == "backward":
            bw = bench_backward(gqa, workloads.LLAMA_PREFILL, S, Wu, torch, 2000)
            log(f"backward: {bw['avg_ms'] * 1e3:.1f} us, {bw['tflops']:.1f} TFLOP/s")
            legs["backward"] = (bw, mfma_roofline(
                bw, "bwd_rowdot + bwd_dkdv_kernel<128, false, 4> + bwd_dq_kernel<128, false>",
                sha_key="backward"),
                prefill_config(workloads.LLAMA_PREFILL))
        elif name == "gva":
            gv = bench_gva(gqa, workloads.GVA_PREFILL, S, Wu, torch, 8000)
            log(f"gva prefill: {gv['avg_ms'] * 1e3:.1f} us, {gv['tflops']:.1f} TFLOP/s")
            cfg = prefill_config(workloads.GVA_PREFILL)
            cfg.update({"H": cfg.pop("Hkv"), "HV": cfg.pop("Hq")})
            legs["gva"] = (gv, mfma_roofline(gv, "prefill_pp_kernel<64, 128, false, false, "
                                                 "false>", "gva"), cfg)
        elif name == "decode":
            run_decode("decode", workloads.DECODE, 3000)
        elif name == "ragged":
            run_decode("ragged", workloads.RAGGED_DECODE, 7000)
        elif name == "longdecode":
            run_decode("longdecode", workloads.LONG_DECODE, 9000)
        elif name == "windowcache":
            run_decode("windowcache", workloads.WINDOW_CACHE_DECODE, 9500)

    head_key = {"prefill": "prefill"}.get(headline, headline)
    res, roofline, config = legs.pop(head_key)
    if "tflops" in res:
        value, unit = res["tflops"], "TFLOP/s"
    else:
        value, unit = res["gbs"], "GB/s"
    line = {"metric": "GQA prefill TFLOPS (% MFMA peak); decode KV GB/s (% HBM peak)",
            "value": value, "unit": unit, "n_gpus": 1, "steps": S, "warmup": Wu,
            "ms_per_step": res["avg_ms"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) on device)",
            "config": config, "roofline": roofline}
    if legs:
        line["secondary"] = {name: dict(res, roofline=rf, config=cfg)
                             for name, (res, rf, cfg) in legs.items()}
    line["cpu_baseline"] = None
    if not args.no_cpu_baseline and head_key in tensors:
        log("cpu baseline: fp64 oracle on a sample")
        w, t = tensors[head_key]
        line["cpu_baseline"] = cpu_baseline(w, t, torch)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
