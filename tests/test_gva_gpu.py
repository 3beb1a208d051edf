"""GPU parity for grouped value attention (K3 notes, section 4, GVA): H query/key heads shared by
HV = G*H value heads, value head j attended with query/key head j // G. The HIP kernel, called
through the C ABI, is compared element by element with the fp64 oracle (which materialises the
notes' repeat_interleave of q and k). Covered: value rows split into one and several 128-column
slices, slices of one value head (G*d not a multiple of 128), G = 1 (multi-head), d = 64 and 128,
Tq < Tkv, a window with sinks, a packed batch, the log-sum-exp output."""
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


GVA_CASES = [
    # B, Tq, Tkv, H, HV, d, causal, window, n_sink
    (1, 300, 300, 4, 8, 64, True, 0, 0),      # G*d = 128: the scores once per query/key head
    (1, 200, 200, 2, 8, 64, True, 0, 0),      # G*d = 256: two 128-column slices
    (2, 130, 130, 4, 8, 128, False, 0, 0),    # d = 128, G = 2: two slices, not causal
    (1, 77, 333, 2, 6, 64, True, 0, 0),       # G = 3, G*d = 192: one slice per value head
    (1, 257, 257, 8, 8, 128, True, 0, 0),     # G = 1: multi-head attention
    (1, 500, 500, 4, 8, 64, True, 130, 5),    # sliding window with sinks
    (3, 1, 700, 4, 8, 64, True, 0, 0),        # one query row per sequence (a decode step)
]


@pytest.mark.parametrize("case", GVA_CASES,
                         ids=lambda c: "B{}_Tq{}_Tkv{}_H{}_HV{}_d{}_c{}_W{}_S{}".format(*c))
def test_bf16_gva_vs_oracle(gqa, orc, case):
    B, Tq, Tkv, H, HV, d, causal, W, S = case
    say(f"bf16 gva {case}")
    q = workloads.randn_bf16((B, Tq, H, d), 141)
    k = workloads.randn_bf16((B, Tkv, H, d), 142)
    v = workloads.randn_bf16((B, Tkv, HV, d), 143)
    out = gqa.gqa_attn_prefill_gva(to_dev(q), to_dev(k), to_dev(v), causal=causal, window=W,
                                   n_sink=S)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (B, Tq, HV, d)
    ref = orc.attention_gva(host_view(q), host_view(k), host_view(v), causal=causal, window=W,
                            n_sink=S)
    assert_bf16_close(to_f64(out), ref, what=str(case))


def test_bf16_gva_packed_vs_oracle(gqa, orc):
    lens = (300, 1, 129, 64)
    say(f"bf16 gva packed {lens}")
    tot = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = workloads.randn_bf16((1, tot, 4, 64), 144)
    k = workloads.randn_bf16((1, tot, 4, 64), 145)
    v = workloads.randn_bf16((1, tot, 8, 64), 146)
    out = gqa.gqa_attn_prefill_gva(to_dev(q), to_dev(k), to_dev(v), causal=True,
                                   cu_seqlens=to_dev(cu), max_seqlen=max(lens))
    torch.cuda.synchronize()
    ref = orc.attention_gva(host_view(q), host_view(k), host_view(v), causal=True, cu_seqlens=cu)
    assert_bf16_close(to_f64(out), ref, what="packed gva")


def test_bf16_gva_single_group_member_is_mha(gqa):
    """G = 1 runs the multi-head configuration of the same kernel: bit-identical to
    gqa_attn_prefill with Hq = Hkv."""
    say("bf16 gva G=1 == mha")
    q = to_dev(workloads.randn_bf16((2, 190, 4, 128), 147))
    k = to_dev(workloads.randn_bf16((2, 190, 4, 128), 148))
    v = to_dev(workloads.randn_bf16((2, 190, 4, 128), 149))
    a = gqa.gqa_attn_prefill_gva(q, k, v, causal=True)
    b = gqa.gqa_attn_prefill(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_bf16_gva_lse_matches_the_shared_scores(gqa):
    """The log-sum-exp of a query/key head depends on q and k only: the value-grouped call and a
    multi-head call on the same q, k (any values) agree."""
    say("bf16 gva lse")
    B, T, H, G, d = 1, 300, 4, 2, 64
    q = to_dev(workloads.randn_bf16((B, T, H, d), 150))
    k = to_dev(workloads.randn_bf16((B, T, H, d), 151))
    v = to_dev(workloads.randn_bf16((B, T, H * G, d), 152))
    l1 = torch.empty(B, T, H, dtype=torch.float32, device="cuda")
    l2 = torch.empty_like(l1)
    gqa.gqa_attn_prefill_gva(q, k, v, causal=True, lse=l1)
    gqa.gqa_attn_prefill_ex(q, k, v[:, :, :H].contiguous(), causal=True, lse=l2)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(l1 - l2)).item() <= 1e-5
