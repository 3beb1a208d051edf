"""Host-side checks of bench.py (no GPU): the one-GPU contract and the algorithmic work counts
its roofline divides by.

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
