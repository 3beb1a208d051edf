"""GPU parity for decode against caches bounded to the sliding window (course page "Week 7.
Attention", step 3: the window bounds the cache to its size, and the sink tokens are never dropped).
Each sequence's cache holds n_sink + window slots; its entry counts (which may exceed that) are
on the device. The HIP kernels, called through the C ABI, are compared element by element with
the fp64 oracle, which reads every visible entry back from its slot; the cases cover empty caches,
lengths below the sinks, exactly at the capacity and far past it, windows of one entry, more sinks
than window slots, splits of one sequence over many workgroups, two chunks of query heads, the
balanced order of many sequences, and the query's rotary turn and QK-norm. One case checks that the
bounded cache gives bit for bit the output of the windowed decode of the whole cache."""
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


CASES = [
    # B, window, n_sink, Hq, Hkv, d, entry counts
    (4, 64, 4, 32, 8, 128, (0, 3, 68, 1000)),         # empty, below the sinks, full, wrapped
    (3, 100, 0, 8, 2, 64, (50, 100, 12345)),          # no sinks, d = 64
    (2, 4096, 4, 16, 1, 128, (5000, 100000)),         # one sequence split over 16 workgroups
    (5, 33, 70, 40, 2, 128, (1, 69, 70, 103, 5000)),  # more sinks than window slots, G = 20
    (1, 1, 0, 8, 8, 128, (10,)),                      # a window of one entry
    (1, 1, 3, 4, 1, 64, (2, )),                       # fewer entries than sinks
    (300, 40, 2, 8, 2, 64, tuple((i * 97) % 500 for i in range(300))),  # balanced order
]


def _ring_inputs(B, W, S, Hq, Hkv, d, seed):
    q = workloads.randn_bf16((B, 1, Hq, d), seed)
    k = workloads.randn_bf16((B, S + W, Hkv, d), seed + 1)
    v = workloads.randn_bf16((B, S + W, Hkv, d), seed + 2)
    return q, k, v


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_W{}_S{}_Hq{}_Hkv{}_d{}".format(*c[:6]))
def test_window_cache_decode_vs_oracle(gqa, orc, case):
    B, W, S, Hq, Hkv, d, lens = case
    say(f"window-cache decode B={B} W={W} S={S} Hq={Hq} Hkv={Hkv} d={d}")
    q, k, v = _ring_inputs(B, W, S, Hq, Hkv, d, 61)
    lens_dev = to_dev(np.asarray(lens, dtype=np.int32))
    out = gqa.gqa_attn_decode_window_cache(to_dev(q), to_dev(k), to_dev(v), lens_dev, window=W,
                                           n_sink=S)
    torch.cuda.synchronize()
    got = to_f64(out)
    qh = host_view(q)
    kc = oracle.unroll_window_cache(host_view(k), lens, W, S, compact=True)
    vc = oracle.unroll_window_cache(host_view(v), lens, W, S, compact=True)
    for b, L in enumerate(lens):
        if L == 0:   # nothing visible: the zero row
            assert np.array_equal(got[b], np.zeros_like(got[b])), f"seq {b}: empty cache"
            continue
        # the visible entries alone, in arrival order: plain attention over all of them
        ref = orc.attention(qh[b:b + 1], kc[b], vc[b])
        assert_bf16_close(got[b:b + 1], ref, what=f"{case[:6]} seq {b} len {L}")


@pytest.mark.parametrize("mode", ["rope", "rope_qknorm"])
def test_window_cache_decode_rope_and_norm(gqa, orc, mode):
    """The query turned at its position (entry count - 1) and normalised; the cache holds keys
    turned at their own positions when they were written."""
    B, W, S, Hq, Hkv, d, lens = 3, 48, 4, 32, 8, 128, (10, 100, 700)
    say(f"window-cache decode {mode}")
    q, k, v = _ring_inputs(B, W, S, Hq, Hkv, d, 71)
    cos, sin = workloads.rope_tables(1024, d)
    rope = (to_dev(cos), to_dev(sin))
    norm, norm_dev = None, None
    if mode == "rope_qknorm":
        wq = (1.0 + 0.1 * np.random.default_rng(72).standard_normal(d)).astype(np.float32)
        norm = (wq, np.ones(d, dtype=np.float32), 1e-6)
        norm_dev = (to_dev(wq), None, 1e-6)
    out = gqa.gqa_attn_decode_window_cache(to_dev(q), to_dev(k), to_dev(v),
                                           to_dev(np.asarray(lens, dtype=np.int32)), window=W,
                                           n_sink=S, rope=rope, qk_norm=norm_dev)
    torch.cuda.synchronize()
    got = to_f64(out)
    qh = host_view(q)
    ku = oracle.unroll_window_cache(host_view(k), lens, W, S)
    vu = oracle.unroll_window_cache(host_view(v), lens, W, S)
    for b, L in enumerate(lens):
        ref = orc.attention(qh[b:b + 1], ku[b], vu[b], causal=True, window=W, n_sink=S,
                            rope=(cos, sin), rope_mode="q", qk_norm=norm, qk_norm_mode="q")
        assert_bf16_close(got[b:b + 1], ref, what=f"{mode} seq {b} len {L}")


def test_window_cache_matches_windowed_decode_of_whole_cache(gqa):
    """Whole caches of up to 3000 entries copied into bounded caches slot by slot: the bounded
    decode reads the same visible entries in the same order as the windowed decode of the whole
    cache (one split each at this shape), so the outputs are identical."""
    B, W, S, Hq, Hkv, d, Tmax = 128, 256, 4, 8, 2, 64, 3000
    say("window-cache decode vs windowed decode of the whole cache")
    rng = np.random.default_rng(81)
    lens = rng.integers(0, Tmax + 1, size=B).astype(np.int32)
    lens[:4] = (0, 1, S + W, Tmax)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(82)
    q = torch.randn(B, 1, Hq, d, generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn(B, Tmax, Hkv, d, generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn(B, Tmax, Hkv, d, generator=gen, device="cuda").to(torch.bfloat16)
    # slot s of sequence b holds the newest entry e < lens[b] with slot(e) = s (entries of a
    # sequence are written in order, each over the one `window` places before it)
    entries = np.arange(Tmax)
    slots = np.where(entries < S, entries, S + (entries - S) % W)
    src = np.zeros((B, S + W), dtype=np.int64)
    for b in range(B):
        for e in range(int(lens[b])):
            src[b, slots[e]] = e
    idx = torch.from_numpy(src).cuda()[:, :, None, None].expand(B, S + W, Hkv, d)
    kr = torch.gather(k, 1, idx).contiguous()
    vr = torch.gather(v, 1, idx).contiguous()
    lens_dev = to_dev(lens)
    a = gqa.gqa_attn_decode_window_cache(q, kr, vr, lens_dev, window=W, n_sink=S)
    b_ = gqa.gqa_attn_decode_ex(q, k, v, cache_lens=lens_dev, window=W, n_sink=S)
    torch.cuda.synchronize()
    assert torch.equal(a, b_)
