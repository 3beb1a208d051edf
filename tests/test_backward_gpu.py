"""GPU parity for the backward kernels (dq, dk, dv of sum(out * dout)) against the fp64 oracle's
chain-rule gradients, including the G-fold sum for shared key/value heads (K3 notes, section 4,
backward). The GPU backward reads the GPU forward's bf16 output and its row log-sum-exp, as a
training step would.

Criterion: max |gpu - oracle| / max |oracle| <= 1e-2 per gradient (the bf16 criterion relative to
the largest value; gradients have no fixed scale, so no absolute bound): bf16 inputs and outputs,
fp32 accumulation, P and dS rounded to bf16 for the matrix cores (2^-9 relative each)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import host_view, say, to_dev, to_f64

pytestmark = pytest.mark.gpu
GRAD_REL = 1e-2


@pytest.fixture(scope="module")
def gqa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_query_softmax_amd as g
    return g


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def _rel(got, ref):
    assert np.all(np.isfinite(got))
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def _check_grads(got, refs, what):
    """Each gradient relative to its own largest value; where the exact gradient is zero
    everywhere (every row sees a single key: P = 1, dS = P (dP - D) = 0, so dq and dk vanish),
    the rounding noise is measured against dv's largest value instead."""
    scale_dv = float(np.max(np.abs(refs[2])))
    for name, gt, ref in zip(("dq", "dk", "dv"), got, refs):
        assert np.all(np.isfinite(gt)), (what, name)
        own = float(np.max(np.abs(ref)))
        e = float(np.max(np.abs(gt - ref))) / (own if own > 0 else scale_dv)
        assert e <= GRAD_REL, f"{what} {name}: rel-to-max {e:.3g} (own max {own:.3g})"


BWD_CASES = [
    # B, Tq, Tkv, Hq, Hkv, d, causal
    (1, 200, 200, 8, 2, 128, True),
    (2, 130, 130, 4, 4, 64, False),     # MHA, d = 64, not causal
    (1, 77, 333, 8, 1, 128, True),      # MQA, Tq < Tkv (bottom-right)
    (1, 64, 64, 6, 2, 128, True),       # G = 3
    (1, 300, 300, 32, 8, 128, True),    # the 32/8 grouping
    (2, 33, 33, 16, 1, 128, False),     # one key past a 32-key chunk
]


@pytest.mark.parametrize("case", BWD_CASES,
                         ids=lambda c: "B{}_Tq{}_Tkv{}_Hq{}_Hkv{}_d{}_c{}".format(*c))
def test_bf16_backward_vs_oracle(gqa, orc, case):
    B, Tq, Tkv, Hq, Hkv, d, causal = case
    say(f"bf16 backward {case}")
    q = workloads.randn_bf16((B, Tq, Hq, d), 131)
    k = workloads.randn_bf16((B, Tkv, Hkv, d), 132)
    v = workloads.randn_bf16((B, Tkv, Hkv, d), 133)
    g = workloads.randn_bf16((B, Tq, Hq, d), 134)
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    lse = torch.empty(B, Tq, Hq, dtype=torch.float32, device="cuda")
    out = gqa.gqa_attn_prefill_ex(qd, kd, vd, causal=causal, lse=lse)
    dq, dk, dv = gqa.gqa_attn_backward(qd, kd, vd, out, gd, lse, causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv = orc.attention_bwd(host_view(q), host_view(k), host_view(v), host_view(g),
                                   causal=causal)
    errs = {name: _rel(to_f64(a), r) for name, a, r in (("dq", dq, rq), ("dk", dk, rk),
                                                        ("dv", dv, rv))}
    say(f"bf16 backward {case}: rel-to-max {errs}")
    assert all(e <= GRAD_REL for e in errs.values()), errs


def test_bf16_forward_lse_consistent(gqa, orc):
    """The row log-sum-exp the forward writes reproduces the oracle's output: with a one-hot value
    table the attention output is the softmax weight itself, exp(s_j - L)."""
    say("bf16 forward lse")
    B, T, Hq, Hkv, d = 1, 96, 4, 2, 128
    q = workloads.randn_bf16((B, T, Hq, d), 135)
    k = workloads.randn_bf16((B, T, Hkv, d), 136)
    v = torch.zeros(B, T, Hkv, d, dtype=torch.bfloat16)
    v[0, 5, :, 0] = 1.0           # out[..., 0] = weight of key 5
    lse = torch.empty(B, T, Hq, dtype=torch.float32, device="cuda")
    gqa.gqa_attn_prefill_ex(to_dev(q), to_dev(k), to_dev(v), causal=True, lse=lse)
    torch.cuda.synchronize()
    w5 = orc.attention(host_view(q), host_view(k), host_view(v), causal=True)[0, :, :, 0]
    # the weight of key 5 is exp(s_5 - L): recover L from the oracle's weight and s_5
    qf = workloads.bits_to_f32(host_view(q)).astype(np.float64)
    kf = workloads.bits_to_f32(host_view(k)).astype(np.float64)
    G = Hq // Hkv
    s5 = np.einsum("thc,hc->th", qf[0], np.repeat(kf[0, 5], G, axis=0)) / np.sqrt(d)
    rows = np.arange(5, T)   # rows that see key 5
    L_ref = s5[rows] - np.log(w5[rows])
    L_gpu = lse.cpu().numpy()[0, rows]
    assert np.max(np.abs(L_gpu - L_ref)) <= 2e-2, np.max(np.abs(L_gpu - L_ref))


WINDOW_BWD_CASES = [
    # B, Tq, Tkv, Hq, Hkv, d, window, n_sink  (course page "Week 7. Attention", step 3)
    (1, 300, 300, 8, 2, 128, 64, 0),     # window edge inside key tiles and query chunks
    (2, 200, 257, 16, 4, 64, 33, 5),     # Tq < Tkv, sinks below the window
    (1, 150, 150, 32, 1, 128, 1, 0),     # one-key window: each row sees only its own key
    (1, 129, 129, 4, 4, 128, 200, 2),    # window wider than the sequence (plain causal)
    (1, 500, 500, 8, 2, 128, 100, 70),   # sinks spanning more than one 64-key tile
]


@pytest.mark.parametrize("case", WINDOW_BWD_CASES,
                         ids=lambda c: "B{}_Tq{}_Tkv{}_Hq{}_Hkv{}_d{}_W{}_S{}".format(*c))
def test_bf16_backward_window_vs_oracle(gqa, orc, case):
    """Backward of the sliding-window forward (with sinks) against the oracle's windowed
    chain-rule gradients; the forward runs with the same window and writes the log-sum-exp."""
    B, Tq, Tkv, Hq, Hkv, d, W, S = case
    say(f"bf16 backward window {case}")
    q = workloads.randn_bf16((B, Tq, Hq, d), 141)
    k = workloads.randn_bf16((B, Tkv, Hkv, d), 142)
    v = workloads.randn_bf16((B, Tkv, Hkv, d), 143)
    g = workloads.randn_bf16((B, Tq, Hq, d), 144)
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    lse = torch.empty(B, Tq, Hq, dtype=torch.float32, device="cuda")
    out = gqa.gqa_attn_prefill_ex(qd, kd, vd, causal=True, window=W, n_sink=S, lse=lse)
    dq, dk, dv = gqa.gqa_attn_backward(qd, kd, vd, out, gd, lse, causal=True, window=W, n_sink=S)
    torch.cuda.synchronize()
    refs = orc.attention_bwd(host_view(q), host_view(k), host_view(v), host_view(g), causal=True,
                             window=W, n_sink=S)
    _check_grads([to_f64(x) for x in (dq, dk, dv)], refs, str(case))


PACKED_BWD_CASES = [
    # sequence lengths, Hq, Hkv, d, window, n_sink
    ((130, 1, 64, 257), 8, 2, 128, 0, 0),
    ((70, 0, 200, 33), 16, 4, 64, 0, 0),      # an empty sequence
    ((300, 150), 8, 1, 128, 48, 3),           # packed with a window and sinks
]


@pytest.mark.parametrize("case", PACKED_BWD_CASES, ids=lambda c: f"lens{len(c[0])}_Hq{c[1]}_W{c[4]}")
def test_bf16_backward_packed_vs_oracle(gqa, orc, case):
    """Backward of a packed batch: each sequence's gradients against the oracle run on that
    sequence alone (sequences do not attend to each other, so their gradients are separate)."""
    lens, Hq, Hkv, d, W, S = case
    say(f"bf16 backward packed {case}")
    tot = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = workloads.randn_bf16((1, tot, Hq, d), 151)
    k = workloads.randn_bf16((1, tot, Hkv, d), 152)
    v = workloads.randn_bf16((1, tot, Hkv, d), 153)
    g = workloads.randn_bf16((1, tot, Hq, d), 154)
    qd, kd, vd, gd, cud = to_dev(q), to_dev(k), to_dev(v), to_dev(g), to_dev(cu)
    lse = torch.empty(1, tot, Hq, dtype=torch.float32, device="cuda")
    out = gqa.gqa_attn_prefill_ex(qd, kd, vd, causal=True, window=W, n_sink=S, lse=lse,
                                  cu_seqlens=cud, max_seqlen=max(lens))
    dq, dk, dv = gqa.gqa_attn_backward(qd, kd, vd, out, gd, lse, causal=True, window=W, n_sink=S,
                                       cu_seqlens=cud, max_seqlen=max(lens))
    torch.cuda.synchronize()
    qh, kh, vh, gh = host_view(q), host_view(k), host_view(v), host_view(g)
    got = [to_f64(x) for x in (dq, dk, dv)]
    for s in range(len(lens)):
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:
            continue
        refs = orc.attention_bwd(qh[:, a:b], kh[:, a:b], vh[:, a:b], gh[:, a:b], causal=True,
                                 window=W, n_sink=S)
        _check_grads([gt[:, a:b] for gt in got], refs, f"{case} seq {s}")
