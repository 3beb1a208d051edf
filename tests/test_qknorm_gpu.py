"""GPU parity for QK-norm fused into the attention kernels (course page "Week 7. Attention",
step 3: RMSNorm of q and k before the dot product), alone and followed by the rotary embedding:
prefill normalises queries at load and keys while staging them; decode normalises the query
against a cache of processed keys. Compared element by element with the fp64 oracle, which
normalises the same bf16 inputs with the same fp32 weights in double precision."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_bf16_close, host_view, say, to_dev, to_f64

pytestmark = pytest.mark.gpu
EPS = 1e-6


@pytest.fixture(scope="module")
def gqa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_query_softmax_amd as g
    return g


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def _weights(d, seed):
    rng = np.random.default_rng(seed)
    wq = (rng.random(d) * 1.5 + 0.25).astype(np.float32)
    wk = (rng.random(d) * 1.5 + 0.25).astype(np.float32)
    return wq, wk


PREFILL_NORM_CASES = [
    # B, Tq, Tkv, Hq, Hkv, d, causal, rope, q_scale
    (1, 300, 300, 8, 2, 128, True, False, 1.0),
    (1, 300, 300, 8, 2, 128, True, True, 1.0),
    (2, 200, 200, 32, 1, 128, True, True, 7.0),     # MQA, large-norm queries
    (1, 77, 333, 4, 4, 64, True, True, 0.1),        # Tq < Tkv, d = 64, small-norm queries
    (1, 150, 150, 6, 2, 128, False, False, 1.0),    # not causal, G = 3
    (1, 129, 129, 8, 8, 64, True, False, 1.0),      # MHA, d = 64
]


@pytest.mark.parametrize("case", PREFILL_NORM_CASES,
                         ids=lambda c: "B{}_Tq{}_Tkv{}_Hq{}_Hkv{}_d{}_c{}_rope{}_x{}".format(*c))
def test_bf16_prefill_qknorm_vs_oracle(gqa, orc, case):
    B, Tq, Tkv, Hq, Hkv, d, causal, rope, qs = case
    say(f"bf16 prefill qk-norm {case}")
    q = workloads.to_bf16(workloads.randn_f32((B, Tq, Hq, d), 161) * qs)
    k = workloads.randn_bf16((B, Tkv, Hkv, d), 162)
    v = workloads.randn_bf16((B, Tkv, Hkv, d), 163)
    wq, wk = _weights(d, 164)
    tabs = workloads.rope_tables(Tkv + 3, d) if rope else None
    out = gqa.gqa_attn_prefill_ex(to_dev(q), to_dev(k), to_dev(v), causal=causal,
                                  rope=tuple(to_dev(t) for t in tabs) if rope else None,
                                  qk_norm=(to_dev(wq), to_dev(wk), EPS))
    torch.cuda.synchronize()
    ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=causal, rope=tabs,
                        qk_norm=(wq, wk, EPS))
    assert_bf16_close(to_f64(out), ref, what=str(case))


def test_bf16_prefill_qknorm_packed_window_vs_oracle(gqa, orc):
    lens = (300, 1, 129, 64)
    W, S = 90, 3
    say(f"bf16 prefill qk-norm packed {lens} window {W} sinks {S}")
    tot = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = workloads.randn_bf16((1, tot, 16, 128), 165)
    k = workloads.randn_bf16((1, tot, 4, 128), 166)
    v = workloads.randn_bf16((1, tot, 4, 128), 167)
    wq, wk = _weights(128, 168)
    tabs = workloads.rope_tables(max(lens), 128)
    out = gqa.gqa_attn_prefill_ex(to_dev(q), to_dev(k), to_dev(v), causal=True, window=W,
                                  n_sink=S, rope=tuple(to_dev(t) for t in tabs),
                                  qk_norm=(to_dev(wq), to_dev(wk), EPS), cu_seqlens=to_dev(cu),
                                  max_seqlen=max(lens))
    torch.cuda.synchronize()
    ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=True, window=W,
                        n_sink=S, cu_seqlens=cu, rope=tabs, qk_norm=(wq, wk, EPS))
    assert_bf16_close(to_f64(out), ref, what="packed qk-norm")


def test_bf16_prefill_qknorm_scale_invariant(gqa):
    """QK-norm fixes the logit scale: scaling q by 4 and k by 1/8 (exact in bf16) changes the
    output only through eps, far below bf16 resolution."""
    say("bf16 prefill qk-norm scale invariance")
    q = workloads.randn_bf16((1, 200, 8, 128), 169)
    k = workloads.randn_bf16((1, 200, 2, 128), 170)
    v = to_dev(workloads.randn_bf16((1, 200, 2, 128), 171))
    wq, wk = (to_dev(w) for w in _weights(128, 172))
    a = gqa.gqa_attn_prefill_ex(to_dev(q), to_dev(k), v, causal=True, qk_norm=(wq, wk, EPS))
    b = gqa.gqa_attn_prefill_ex(to_dev(q * 4), to_dev(k * 0.125), v, causal=True,
                                qk_norm=(wq, wk, EPS))
    torch.cuda.synchronize()
    assert torch.max(torch.abs(a.float() - b.float())).item() <= 2 ** -7


DECODE_NORM_CASES = [
    # B, Tmax, Hq, Hkv, d, lens, rope
    (4, 2000, 32, 8, 128, None, True),
    (3, 700, 8, 2, 128, (700, 33, 1), False),
    (2, 3000, 16, 1, 64, (2999, 1500), True),
]


@pytest.mark.parametrize("case", DECODE_NORM_CASES,
                         ids=lambda c: "B{}_Tmax{}_Hq{}_Hkv{}_d{}_rope{}".format(*c[:5], c[6]))
def test_bf16_decode_qknorm_vs_oracle(gqa, orc, case):
    B, Tmax, Hq, Hkv, d, lens, rope = case
    say(f"bf16 decode qk-norm {case[:5]} rope={rope}")
    wq, wk = _weights(d, 173)
    q = workloads.randn_bf16((B, 1, Hq, d), 174)
    k = workloads.randn_bf16((B, Tmax, Hkv, d), 175)
    v = workloads.randn_bf16((B, Tmax, Hkv, d), 176)
    tabs = workloads.rope_tables(Tmax, d) if rope else None
    # the cache a model with QK-norm (and RoPE) writes: keys normalised (and turned), in float64,
    # rounded to bf16
    x = k.double()
    x = x * torch.rsqrt((x * x).mean(-1, keepdim=True) + EPS) * torch.from_numpy(wk).double()
    if rope:
        z = torch.view_as_complex(x.reshape(B, Tmax, Hkv, d // 2, 2).contiguous())
        rot = torch.complex(torch.from_numpy(tabs[0]).double(), torch.from_numpy(tabs[1]).double())
        x = torch.view_as_real(z * rot[None, :, None, :]).reshape(B, Tmax, Hkv, d)
    kc = x.to(torch.bfloat16)
    lens_dev = to_dev(np.asarray(lens, dtype=np.int32)) if lens else None
    out = gqa.gqa_attn_decode_ex(to_dev(q), to_dev(kc), to_dev(v), cache_lens=lens_dev,
                                 rope=tuple(to_dev(t) for t in tabs) if rope else None,
                                 qk_norm=(to_dev(wq), to_dev(wk), EPS))
    torch.cuda.synchronize()
    got = to_f64(out)
    qh, kh, vh = host_view(q), host_view(kc), host_view(v)
    for b in range(B):
        L = lens[b] if lens else Tmax
        ref = orc.attention(qh[b:b + 1], np.ascontiguousarray(kh[b:b + 1, :L]),
                            np.ascontiguousarray(vh[b:b + 1, :L]), causal=True, rope=tabs,
                            rope_mode="q", qk_norm=(wq, wk, EPS), qk_norm_mode="q")
        assert_bf16_close(got[b:b + 1], ref, what=f"{case[:5]} seq {b} len {L}")


def _ref_prepared(k_bf16, tabs, wk, pos0=0, lens=None):
    """Keys normalised (wk not None) and turned (tabs not None) in float64 (per sequence
    positions pos0 + j), as float64 numpy."""
    x = k_bf16.double()
    if wk is not None:
        x = x * torch.rsqrt((x * x).mean(-1, keepdim=True) + EPS) * torch.from_numpy(wk).double()
    if tabs is not None:
        B, T, H, d = x.shape
        if lens is None:
            pos = torch.arange(T) + pos0
        else:
            pos = torch.cat([torch.arange(n) for n in lens]) + pos0
        z = torch.view_as_complex(x.reshape(B, T, H, d // 2, 2).contiguous())
        rot = torch.complex(torch.from_numpy(tabs[0]).double(), torch.from_numpy(tabs[1]).double())
        x = torch.view_as_real(z * rot[pos][None, :, None, :]).reshape(B, T, H, d)
    return x.numpy()


PREP_CASES = [
    # B, T, H, d, norm, rope, pos0, packed lens
    (2, 300, 8, 128, True, True, 0, None),
    (2, 300, 8, 128, False, True, 5, None),
    (1, 77, 2, 64, True, False, 0, None),
    (1, 494, 4, 128, True, True, 3, (300, 1, 129, 64)),
]


@pytest.mark.parametrize("case", PREP_CASES,
                         ids=lambda c: "B{}_T{}_H{}_d{}_norm{}_rope{}_p{}_packed{}".format(
                             *c[:7], c[7] is not None))
def test_bf16_prepare_keys_vs_float64(gqa, case):
    B, T, H, d, norm, rope, pos0, lens = case
    say(f"bf16 prepare keys {case}")
    k = workloads.randn_bf16((B, T, H, d), 177)
    wq, wk = _weights(d, 178)
    tabs = workloads.rope_tables(T + pos0 + 1, d) if rope else None
    cu = None
    if lens is not None:
        cu = to_dev(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    got = gqa.gqa_prepare_keys(to_dev(k), rope=tuple(to_dev(t) for t in tabs) if rope else None,
                               qk_norm=(None, to_dev(wk), EPS) if norm else None, pos0=pos0,
                               cu_seqlens=cu, max_seqlen=max(lens) if lens is not None else None)
    torch.cuda.synchronize()
    ref = _ref_prepared(k, tabs, wk if norm else None, pos0, lens)
    # one rounding to bf16 of an fp32 computation: within 2^-8 of each value (+ tiny absolute)
    err = np.abs(to_f64(got) - ref) - (2.0 ** -8 * np.abs(ref) + 1e-6)
    assert np.max(err) <= 0, np.max(err)


PREPARED_PREFILL_CASES = [
    # B, Tq, Tkv, Hq, Hkv, d, rope, norm
    (1, 300, 300, 8, 2, 128, True, True),
    (2, 200, 200, 32, 1, 128, True, False),
    (1, 77, 333, 4, 4, 64, True, True),
    (1, 150, 150, 6, 2, 128, False, True),
]


@pytest.mark.parametrize("case", PREPARED_PREFILL_CASES,
                         ids=lambda c: "B{}_Tq{}_Tkv{}_Hq{}_Hkv{}_d{}_rope{}_norm{}".format(*c))
def test_bf16_prefill_keys_prepared_vs_oracle(gqa, orc, case):
    """gqa_prepare_keys then the attention with keys_prepared equals the oracle's full
    processing of the raw q, k."""
    B, Tq, Tkv, Hq, Hkv, d, rope, norm = case
    say(f"bf16 prefill keys prepared {case}")
    q = workloads.randn_bf16((B, Tq, Hq, d), 179)
    k = workloads.randn_bf16((B, Tkv, Hkv, d), 180)
    v = workloads.randn_bf16((B, Tkv, Hkv, d), 181)
    wq, wk = _weights(d, 182)
    tabs = workloads.rope_tables(Tkv, d) if rope else None
    dt = tuple(to_dev(t) for t in tabs) if rope else None
    qn = (to_dev(wq), to_dev(wk), EPS) if norm else None
    kp = gqa.gqa_prepare_keys(to_dev(k), rope=dt, qk_norm=qn)
    out = gqa.gqa_attn_prefill_ex(to_dev(q), kp, to_dev(v), causal=True, rope=dt,
                                  qk_norm=(qn[0], None, EPS) if norm else None,
                                  keys_prepared=True)
    torch.cuda.synchronize()
    ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=True, rope=tabs,
                        qk_norm=(wq, wk, EPS) if norm else None)
    assert_bf16_close(to_f64(out), ref, what=str(case))


def test_bf16_decode_with_prepared_cache_vs_oracle(gqa, orc):
    """A cache written by gqa_prepare_keys (QK-norm and RoPE) serves decode."""
    B, Tmax, Hq, Hkv, d = 3, 1500, 32, 8, 128
    lens = (1500, 700, 1)
    say("bf16 decode with a prepared cache")
    wq, wk = _weights(d, 183)
    tabs = workloads.rope_tables(Tmax, d)
    q = workloads.randn_bf16((B, 1, Hq, d), 184)
    k = workloads.randn_bf16((B, Tmax, Hkv, d), 185)
    v = workloads.randn_bf16((B, Tmax, Hkv, d), 186)
    dt = tuple(to_dev(t) for t in tabs)
    kc = gqa.gqa_prepare_keys(to_dev(k), rope=dt, qk_norm=(None, to_dev(wk), EPS))
    out = gqa.gqa_attn_decode_ex(to_dev(q), kc, to_dev(v),
                                 cache_lens=to_dev(np.asarray(lens, dtype=np.int32)), rope=dt,
                                 qk_norm=(to_dev(wq), None, EPS))
    torch.cuda.synchronize()
    got = to_f64(out)
    qh, kh, vh = host_view(q), host_view(k), host_view(v)
    for b in range(B):
        L = lens[b]
        ref = orc.attention(qh[b:b + 1], np.ascontiguousarray(kh[b:b + 1, :L]),
                            np.ascontiguousarray(vh[b:b + 1, :L]), causal=True, rope=tabs,
                            qk_norm=(wq, wk, EPS))
        assert_bf16_close(got[b:b + 1], ref, what=f"seq {b} len {L}")
