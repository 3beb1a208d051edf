"""GPU parity for the mask and cache variants: causal sliding windows with attention sinks in
prefill and decode, and decode against ragged (per-sequence length) caches (course page
"Week 7. Attention", step 3). The HIP kernels, called through the C ABI, are compared element by
element with the fp64 oracle on seeded inputs; windows of one key, windows wider than the
sequence, sinks spanning several key tiles, window edges off the tile grid, empty cache splits and
length-one caches are covered."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_bf16_close, host_view, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gqa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_query_softmax_amd as g
    return g


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


PREFILL_WINDOW_CASES = [
    # B, Tq, Tkv, Hq, Hkv, d, window, n_sink
    (1, 300, 300, 8, 2, 128, 64, 0),      # window one key tile wide
    (2, 200, 200, 8, 2, 128, 50, 4),      # window edge off the tile grid, a few sinks
    (1, 77, 333, 4, 4, 64, 100, 1),       # Tq < Tkv (bottom-right), MHA, d = 64
    (1, 257, 257, 32, 1, 128, 1, 0),      # one-key window: every query sees only itself
    (1, 500, 500, 8, 8, 128, 130, 70),    # sinks over two key tiles, gap before the window
    (1, 150, 150, 6, 2, 128, 1000, 0),    # window wider than the sequence (G = 3)
    (3, 129, 129, 16, 4, 128, 33, 200),   # sinks cover the whole past: plain causal
]


@pytest.mark.parametrize("case", PREFILL_WINDOW_CASES,
                         ids=lambda c: "B{}_Tq{}_Tkv{}_Hq{}_Hkv{}_d{}_W{}_S{}".format(*c))
def test_bf16_prefill_window_vs_oracle(gqa, orc, case):
    B, Tq, Tkv, Hq, Hkv, d, W, S = case
    say(f"bf16 prefill window {case}")
    q = workloads.randn_bf16((B, Tq, Hq, d), 81)
    k = workloads.randn_bf16((B, Tkv, Hkv, d), 82)
    v = workloads.randn_bf16((B, Tkv, Hkv, d), 83)
    out = gqa.gqa_attn_prefill_window(to_dev(q), to_dev(k), to_dev(v), window=W, n_sink=S)
    torch.cuda.synchronize()
    ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=True, window=W,
                        n_sink=S)
    assert_bf16_close(to_f64(out), ref, what=str(case))


def test_bf16_prefill_window_packed_vs_oracle(gqa, orc):
    lens = (700, 64, 1, 333)
    W, S = 96, 3
    say(f"bf16 prefill window packed {lens} W={W} S={S}")
    tot = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = workloads.randn_bf16((1, tot, 16, 128), 84)
    k = workloads.randn_bf16((1, tot, 2, 128), 85)
    v = workloads.randn_bf16((1, tot, 2, 128), 86)
    out = gqa.gqa_attn_prefill_window(to_dev(q), to_dev(k), to_dev(v), window=W, n_sink=S,
                                      cu_seqlens=to_dev(cu), max_seqlen=max(lens))
    torch.cuda.synchronize()
    ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=True, window=W,
                        n_sink=S, cu_seqlens=cu)
    assert_bf16_close(to_f64(out), ref, what="packed window")


def test_bf16_prefill_window_limits_are_exact(gqa):
    """window 0, or a window covering every key, runs the same tiles with the same arithmetic as
    the plain causal call: the outputs are bit-identical."""
    say("bf16 prefill window limits")
    q = to_dev(workloads.randn_bf16((2, 190, 8, 128), 87))
    k = to_dev(workloads.randn_bf16((2, 190, 2, 128), 88))
    v = to_dev(workloads.randn_bf16((2, 190, 2, 128), 89))
    base = gqa.gqa_attn_prefill(q, k, v, causal=True)
    for W, S in ((0, 0), (190, 0), (5000, 7)):
        got = gqa.gqa_attn_prefill_window(q, k, v, window=W, n_sink=S)
        torch.cuda.synchronize()
        assert torch.equal(got, base), (W, S)


DECODE_RAGGED_CASES = [
    # B, Tmax, Hq, Hkv, d, lens, window, n_sink
    (5, 3000, 32, 8, 128, (1, 17, 1000, 2999, 3000), 0, 0),
    (5, 3000, 32, 8, 128, (1, 17, 1000, 2999, 3000), 256, 4),
    (3, 700, 8, 2, 128, (700, 33, 400), 1, 0),
    (3, 700, 8, 2, 128, (700, 33, 400), 65, 70),
    (2, 8192, 16, 1, 64, (5000, 8192), 1000, 16),   # cache splits past the visible entries
    (2, 5000, 40, 2, 128, (4321, 77), 300, 2),       # two chunks of query heads
    # empty caches (length 0: the zero row), with one split per sequence and with several
    (4, 600, 32, 8, 128, (0, 1, 0, 600), 0, 0),
    (2, 9000, 16, 2, 64, (0, 8999), 0, 0),
    (3, 4000, 32, 8, 128, (0, 3000, 17), 512, 3),
    # many sequences: up to 512 their work goes out in a balanced order (ranked by length, ties
    # by index, rows snaking), more than 512 in launch order
    (300, 96, 8, 2, 64, tuple((i % 7) * 13 for i in range(300)), 0, 0),
    (600, 96, 8, 2, 64, tuple((i * 37) % 97 for i in range(600)), 40, 2),
    (130, 3000, 32, 4, 128, tuple((i * 613) % 3001 for i in range(130)), 0, 0),
]


@pytest.mark.parametrize("case", DECODE_RAGGED_CASES,
                         ids=lambda c: "B{}_Tmax{}_Hq{}_Hkv{}_d{}_W{}_S{}".format(*c[:5], *c[6:]))
def test_bf16_decode_ragged_vs_oracle(gqa, orc, case):
    B, Tmax, Hq, Hkv, d, lens, W, S = case
    say(f"bf16 decode ragged {case[:5]} W={W} S={S}")
    q = workloads.randn_bf16((B, 1, Hq, d), 91)
    k = workloads.randn_bf16((B, Tmax, Hkv, d), 92)
    v = workloads.randn_bf16((B, Tmax, Hkv, d), 93)
    lens_dev = to_dev(np.asarray(lens, dtype=np.int32))
    out = gqa.gqa_attn_decode_ragged(to_dev(q), to_dev(k), to_dev(v), cache_lens=lens_dev,
                                     window=W, n_sink=S)
    torch.cuda.synchronize()
    got = to_f64(out)
    qh, kh, vh = host_view(q), host_view(k), host_view(v)
    for b, L in enumerate(lens):
        ref = orc.attention(qh[b:b + 1], np.ascontiguousarray(kh[b:b + 1, :L]),
                            np.ascontiguousarray(vh[b:b + 1, :L]), causal=True, window=W,
                            n_sink=S)
        assert_bf16_close(got[b:b + 1], ref, what=f"{case[:5]} W={W} S={S} seq {b} len {L}")


def test_bf16_decode_ragged_full_is_plain_decode(gqa):
    """No lengths and no window: the same kernel path as gqa_attn_decode, bit-identical."""
    say("bf16 decode ragged == decode")
    q = to_dev(workloads.randn_bf16((4, 1, 32, 128), 94))
    k = to_dev(workloads.randn_bf16((4, 2000, 8, 128), 95))
    v = to_dev(workloads.randn_bf16((4, 2000, 8, 128), 96))
    a = gqa.gqa_attn_decode(q, k, v)
    b = gqa.gqa_attn_decode_ragged(q, k, v)
    full = to_dev(np.full(4, 2000, dtype=np.int32))
    c = gqa.gqa_attn_decode_ragged(q, k, v, cache_lens=full)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_bf16_decode_window_matches_prefill_last_row(gqa):
    """The windowed decode of a cache equals the last row of the windowed prefill over it (both
    kernels agree within the bf16 rounding of their different accumulation orders)."""
    say("bf16 decode window vs prefill window")
    T, W, S = 1500, 200, 5
    q = to_dev(workloads.randn_bf16((2, T, 16, 128), 97))
    k = to_dev(workloads.randn_bf16((2, T, 4, 128), 98))
    v = to_dev(workloads.randn_bf16((2, T, 4, 128), 99))
    pre = gqa.gqa_attn_prefill_window(q, k, v, window=W, n_sink=S)[:, -1:].float()
    dec = gqa.gqa_attn_decode_ragged(q[:, -1:].contiguous(), k, v, window=W, n_sink=S).float()
    torch.cuda.synchronize()
    assert torch.max(torch.abs(pre - dec)).item() <= 2 ** -7 * torch.max(torch.abs(pre)).item()
