"""Host-side checks of bench.py (no GPU): the one-GPU contract, the algorithmic work counts its
roofline divides by, and the rule that a measured HBM traffic figure is reported only for the
kernel sources and the workload its counters were taken on.

The counts are pinned to independent arithmetic: a brute-force count of the visible (query,
key) pairs of small masks, and the closed forms for the benchmark shapes (4·d·Hq flops per
unmasked pair with T(T+1)/2 pairs per causal head; every cached K and V element read once).
"""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("Tq,Tkv", [(1, 1), (5, 5), (7, 19), (1, 33), (16, 16)])
def test_visible_pairs_match_a_brute_force_mask(Tq, Tkv):
    q = np.arange(Tq)[:, None] + (Tkv - Tq)  # bottom-right aligned positions
    k = np.arange(Tkv)[None, :]
    assert bench.visible_pairs(Tq, Tkv, True) == int(np.count_nonzero(k <= q))
    assert bench.visible_pairs(Tq, Tkv, False) == Tq * Tkv


@pytest.mark.parametrize("T,window,n_sink", [(40, 8, 0), (40, 8, 3), (17, 100, 2), (33, 1, 1)])
def test_window_pairs_match_a_brute_force_mask(T, window, n_sink):
    q = np.arange(T)[:, None]
    k = np.arange(T)[None, :]
    vis = (k <= q) & ((k > q - window) | (k < n_sink))
    assert bench.visible_pairs_window(T, window, n_sink) == int(np.count_nonzero(vis))


def test_headline_prefill_flops():
    w = workloads.LLAMA_PREFILL
    assert (w.B, w.Tq, w.Hq, w.d, w.causal) == (1, 4096, 32, 128, True)
    assert bench.prefill_flops(w) == 4 * 128 * 32 * (4096 * 4097 // 2) == 137_472_507_904


def test_packed_prefill_flops_sum_over_sequences():
    w = workloads.VARLEN_PREFILL
    assert w.seqlens == (16384, 8192, 4096, 1024)
    expect = 4 * w.d * w.Hq * sum(n * (n + 1) // 2 for n in w.seqlens)
    assert bench.prefill_flops(w) == expect == 5_790_102_454_272


def test_headline_decode_reads_every_cached_element_once():
    w = workloads.DECODE
    kv_bytes = 2 * w.B * w.Tkv * w.Hkv * w.d * 2
    assert kv_bytes == 2_147_483_648


def _record(tmp_path, sha, workload, nbytes):
    import json
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps({"kernel_source_sha": sha, "workload": workload,
                             "hbm_bytes_per_launch": nbytes}))
    return str(p)


def test_traffic_is_reported_only_for_the_sources_and_workload_it_was_measured_on(
        tmp_path, monkeypatch):
    # the roofline's measured traffic must go null as soon as the kernel's sources change after
    # the counters were taken, and must never be borrowed from another workload's record
    sources = bench.TRAFFIC["prefill"][1]
    sha = bench.kernel_source_sha("prefill")
    name = workloads.LLAMA_PREFILL.name
    monkeypatch.setitem(bench.TRAFFIC, "prefill", (_record(tmp_path, sha, name, 123), sources))
    assert bench.traffic_for("prefill") == 123
    assert bench.traffic_for("prefill", name) == 123
    assert bench.traffic_for("prefill", workloads.MQA_PREFILL.name) is None
    stale = "0" * 16 if sha != "0" * 16 else "1" * 16
    monkeypatch.setitem(bench.TRAFFIC, "prefill", (_record(tmp_path, stale, name, 123), sources))
    assert bench.traffic_for("prefill") is None
    monkeypatch.setitem(bench.TRAFFIC, "prefill", (str(tmp_path / "missing.json"), sources))
    assert bench.traffic_for("prefill") is None


def test_source_hash_follows_every_file_of_the_kernel(tmp_path, monkeypatch):
    # the hash covers each listed source: a change to any one of them (the shared header
    # included) changes it
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    (tmp_path / "a.hip").write_text("kernel a\n")
    (tmp_path / "common.hpp").write_text("shared\n")
    monkeypatch.setitem(bench.TRAFFIC, "probe", ("unused", ("a.hip", "common.hpp")))
    h0 = bench.kernel_source_sha("probe")
    (tmp_path / "common.hpp").write_text("shared, changed\n")
    h1 = bench.kernel_source_sha("probe")
    (tmp_path / "a.hip").write_text("kernel a, changed\n")
    h2 = bench.kernel_source_sha("probe")
    assert len({h0, h1, h2}) == 3 and all(len(h) == 16 for h in (h0, h1, h2))


def test_decode_entries_match_a_brute_force_count():
    """Entries each decode leg reads: for the bounded cache, the entries a query at the last
    position sees (sinks and window) counted one by one."""
    w = workloads.WINDOW_CACHE_DECODE
    assert w.Tkv == w.n_sink + w.window
    seen = sum(int(np.count_nonzero((np.arange(L) < w.n_sink) | (np.arange(L) >= L - w.window)))
               for L in w.cache_lens)
    assert bench.decode_entries(w) == seen == 64 * 4100
    assert bench.decode_entries(workloads.DECODE) == 64 * 8192
    assert bench.decode_entries(workloads.RAGGED_DECODE) == sum(workloads.RAGGED_DECODE.cache_lens)
