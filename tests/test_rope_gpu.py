"""GPU parity for the rotary position embedding fused into the attention kernels (course page
"Week 7. Attention", step 3): prefill turns queries and keys inside the kernel, decode turns the
query and reads a cache of turned keys. Compared element by element with the fp64 oracle, which
turns the same bf16 inputs with the same fp32 tables in double precision."""
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


def _tables(npos, d, base=10000.0):
    c, s = workloads.rope_tables(npos, d, base)
    return (c, s), (to_dev(c), to_dev(s))


PREFILL_ROPE_CASES = [
    # B, Tq, Tkv, Hq, Hkv, d, causal, window, n_sink
    (1, 300, 300, 8, 2, 128, True, 0, 0),
    (2, 200, 200, 32, 1, 128, True, 0, 0),     # MQA
    (1, 77, 333, 4, 4, 64, True, 0, 0),        # Tq < Tkv: queries at positions 256 .. 332
    (1, 150, 150, 6, 2, 128, False, 0, 0),     # not causal, G = 3
    (1, 500, 500, 8, 2, 128, True, 130, 7),    # with a sliding window and sinks
]


@pytest.mark.parametrize("case", PREFILL_ROPE_CASES,
                         ids=lambda c: "B{}_Tq{}_Tkv{}_Hq{}_Hkv{}_d{}_c{}_W{}_S{}".format(*c))
def test_bf16_prefill_rope_vs_oracle(gqa, orc, case):
    B, Tq, Tkv, Hq, Hkv, d, causal, W, S = case
    say(f"bf16 prefill rope {case}")
    q = workloads.randn_bf16((B, Tq, Hq, d), 111)
    k = workloads.randn_bf16((B, Tkv, Hkv, d), 112)
    v = workloads.randn_bf16((B, Tkv, Hkv, d), 113)
    host_t, dev_t = _tables(Tkv + 5, d)
    out = gqa.gqa_attn_prefill_ex(to_dev(q), to_dev(k), to_dev(v), causal=causal, window=W,
                                  n_sink=S, rope=dev_t)
    torch.cuda.synchronize()
    ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=causal, window=W,
                        n_sink=S, rope=host_t)
    assert_bf16_close(to_f64(out), ref, what=str(case))


def test_bf16_prefill_rope_packed_vs_oracle(gqa, orc):
    lens = (300, 1, 129, 64)
    say(f"bf16 prefill rope packed {lens}")
    tot = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = workloads.randn_bf16((1, tot, 16, 128), 114)
    k = workloads.randn_bf16((1, tot, 4, 128), 115)
    v = workloads.randn_bf16((1, tot, 4, 128), 116)
    host_t, dev_t = _tables(max(lens), 128)
    out = gqa.gqa_attn_prefill_ex(to_dev(q), to_dev(k), to_dev(v), causal=True, rope=dev_t,
                                  cu_seqlens=to_dev(cu), max_seqlen=max(lens))
    torch.cuda.synchronize()
    ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=True, cu_seqlens=cu,
                        rope=host_t)
    assert_bf16_close(to_f64(out), ref, what="packed rope")


def test_bf16_prefill_rope_identity_tables_are_exact(gqa):
    """cos = 1, sin = 0 turns nothing: the result is bit-identical to the call without tables."""
    say("bf16 prefill rope identity")
    q = to_dev(workloads.randn_bf16((2, 190, 8, 128), 117))
    k = to_dev(workloads.randn_bf16((2, 190, 2, 128), 118))
    v = to_dev(workloads.randn_bf16((2, 190, 2, 128), 119))
    ones = torch.ones(190, 64, dtype=torch.float32, device="cuda")
    zeros = torch.zeros(190, 64, dtype=torch.float32, device="cuda")
    a = gqa.gqa_attn_prefill(q, k, v, causal=True)
    b = gqa.gqa_attn_prefill_ex(q, k, v, causal=True, rope=(ones, zeros))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _turn_cache(k_bf16, cos_t, sin_t):
    """Keys turned at their positions (the state of a cache written by a RoPE model): complex
    multiplication in float64, rounded to bf16."""
    x = k_bf16.double()
    B, T, H, d = x.shape
    z = torch.view_as_complex(x.reshape(B, T, H, d // 2, 2).contiguous())
    rot = torch.complex(torch.from_numpy(cos_t[:T]).double(), torch.from_numpy(sin_t[:T]).double())
    z = z * rot[None, :, None, :]
    return torch.view_as_real(z).reshape(B, T, H, d).to(torch.bfloat16)


DECODE_ROPE_CASES = [
    # B, Tmax, Hq, Hkv, d, lens, window, n_sink
    (4, 2000, 32, 8, 128, None, 0, 0),
    (3, 700, 8, 2, 128, (700, 33, 1), 0, 0),
    (2, 3000, 16, 1, 64, (2999, 1500), 500, 4),
]


@pytest.mark.parametrize("case", DECODE_ROPE_CASES,
                         ids=lambda c: "B{}_Tmax{}_Hq{}_Hkv{}_d{}_W{}_S{}".format(*c[:5], *c[6:]))
def test_bf16_decode_rope_vs_oracle(gqa, orc, case):
    B, Tmax, Hq, Hkv, d, lens, W, S = case
    say(f"bf16 decode rope {case[:5]} W={W} S={S}")
    cos_t, sin_t = workloads.rope_tables(Tmax, d)
    q = workloads.randn_bf16((B, 1, Hq, d), 121)
    k = _turn_cache(workloads.randn_bf16((B, Tmax, Hkv, d), 122), cos_t, sin_t)
    v = workloads.randn_bf16((B, Tmax, Hkv, d), 123)
    lens_dev = to_dev(np.asarray(lens, dtype=np.int32)) if lens else None
    out = gqa.gqa_attn_decode_ex(to_dev(q), to_dev(k), to_dev(v), cache_lens=lens_dev, window=W,
                                 n_sink=S, rope=(to_dev(cos_t), to_dev(sin_t)))
    torch.cuda.synchronize()
    got = to_f64(out)
    qh, kh, vh = host_view(q), host_view(k), host_view(v)
    for b in range(B):
        L = lens[b] if lens else Tmax
        ref = orc.attention(qh[b:b + 1], np.ascontiguousarray(kh[b:b + 1, :L]),
                            np.ascontiguousarray(vh[b:b + 1, :L]), causal=True, window=W,
                            n_sink=S, rope=(cos_t, sin_t), rope_mode="q")
        assert_bf16_close(got[b:b + 1], ref, what=f"{case[:5]} seq {b} len {L}")
