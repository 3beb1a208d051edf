"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle, element by element,
on seeded inputs small enough for the full oracle yet spanning several tiles and ragged tails.
Plus kernel-level properties that hold exactly (causality, closed forms, determinism)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (assert_bf16_close, assert_f32_close, host_view, say, to_dev, to_f64)

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


# ------------------------------------------------------------------------------------------------
# tiny fp32 lab case: Hkv in {8, 2, 1} by folding (same weights) and by direct generation
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("x1000", [False, True], ids=["unit", "x1000"])
@pytest.mark.parametrize("hkv", [8, 2, 1])
def test_tiny_f32_fold_then_attend(gqa, orc, hkv, x1000):
    say(f"tiny f32 fold->attend hkv={hkv} x1000={x1000}")
    q, k, v = workloads.tiny_lab_inputs(x1000=x1000)
    kd, vd = gqa.gqa_fold_kv(to_dev(k), hkv), gqa.gqa_fold_kv(to_dev(v), hkv)
    out = gqa.gqa_attn_prefill(to_dev(q), kd, vd)
    torch.cuda.synchronize()
    # oracle: fold in fp64, then attention (the lab's heads_out protocol)
    ref = orc.heads_out(q, k, v, hkv)
    atol = 1e-5 * (1000.0 if x1000 else 1.0)   # on the x1000 copy the criterion applies to out/1000
    assert_f32_close(to_f64(out), ref, atol=atol, what=f"hkv={hkv}")
    # the folded K/V themselves
    assert_f32_close(to_f64(kd), orc.fold_kv(k, hkv), atol=1e-5 * (1000 if x1000 else 1))
    if hkv == 8:
        assert np.array_equal(kd.cpu().numpy(), k)   # g = H copies the input


@pytest.mark.parametrize("hkv", [8, 2, 1])
def test_tiny_f32_direct_heads(gqa, orc, hkv):
    say(f"tiny f32 direct hkv={hkv}")
    q, _, _ = workloads.tiny_lab_inputs()
    k, v = workloads.tiny_direct_kv(hkv)
    out = gqa.gqa_attn_prefill(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    assert_f32_close(to_f64(out), orc.attention(q, k, v), what=f"hkv={hkv}")


def test_tiny_f32_g_equals_h_matches_per_head(gqa):
    """g = h is plain multi-head attention: each head computed alone gives the same bits."""
    say("tiny f32 g=h vs per-head")
    q, k, v = (to_dev(a) for a in workloads.tiny_lab_inputs())
    full = gqa.gqa_attn_prefill(q, k, v)
    for i in range(8):
        one = gqa.gqa_attn_prefill(q[:, :, i:i + 1].contiguous(), k[:, :, i:i + 1].contiguous(),
                                   v[:, :, i:i + 1].contiguous())
        assert torch.equal(one[:, :, 0], full[:, :, i]), i


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_f32_head_dims_causal(gqa, orc, d):
    say(f"f32 d={d} causal")
    rng = np.random.default_rng(d)
    q = rng.standard_normal((2, 70, 6, d)).astype(np.float32)
    k = rng.standard_normal((2, 90, 3, d)).astype(np.float32)
    v = rng.standard_normal((2, 90, 3, d)).astype(np.float32)
    out = gqa.gqa_attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=True)
    torch.cuda.synchronize()
    assert_f32_close(to_f64(out), orc.attention(q, k, v, causal=True), what=f"d={d}")


# ------------------------------------------------------------------------------------------------
# bf16 prefill (matrix-core kernel)
# ------------------------------------------------------------------------------------------------

BF16_CASES = [
    # B, Tq, Tkv, Hq, Hkv, d, causal
    (2, 300, 300, 8, 2, 128, True),      # several tiles + ragged tail, G=4
    (2, 300, 300, 8, 2, 128, False),
    (1, 77, 333, 4, 4, 64, True),        # Tq < Tkv, bottom-right causal, MHA
    (1, 77, 333, 4, 4, 64, False),
    (2, 200, 200, 32, 1, 128, True),     # MQA, G=32
    (1, 150, 150, 6, 2, 128, True),      # G=3: columns not a power of two
    (1, 65, 65, 192, 1, 64, True),       # G=192: one head tile of 192 of the 256 columns
    (1, 40, 40, 320, 1, 64, True),       # G=320 > 256 columns: two head tiles (256 + 64 heads)
    (1, 33, 70, 512, 1, 128, False),     # G=512: two full head tiles, one position per tile
    (2, 17, 17, 300, 2, 128, True),      # G=150 per head, two key/value heads
    (3, 1, 513, 16, 4, 128, False),      # one query row per item
    (1, 129, 129, 1, 1, 128, True),      # single head
]


@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: "B{}_Tq{}_Tkv{}_Hq{}_Hkv{}_d{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
def test_bf16_prefill_vs_oracle(gqa, orc, case):
    B, Tq, Tkv, Hq, Hkv, d, causal = case
    say(f"bf16 prefill {case}")
    seed = hash(case) % 1000
    q = workloads.randn_bf16((B, Tq, Hq, d), seed)
    k = workloads.randn_bf16((B, Tkv, Hkv, d), seed + 1)
    v = workloads.randn_bf16((B, Tkv, Hkv, d), seed + 2)
    out = gqa.gqa_attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=causal)
    torch.cuda.synchronize()
    ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=causal)
    assert_bf16_close(to_f64(out), ref, what=str(case))


VARLEN_CASES = [
    ((1, 65, 200, 7, 128), 16, 2, True),
    ((130, 3, 64, 257), 8, 8, True),
    ((33, 100), 32, 1, False),
    ((5, 0, 70, 1, 0), 8, 2, True),   # empty sequences (repeated offsets) and a single token
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: f"lens{len(c[0])}_Hq{c[1]}_Hkv{c[2]}")
def test_bf16_varlen_vs_oracle(gqa, orc, case):
    lens, Hq, Hkv, causal = case
    say(f"bf16 varlen {case}")
    tot = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = workloads.randn_bf16((1, tot, Hq, 128), 11)
    k = workloads.randn_bf16((1, tot, Hkv, 128), 12)
    v = workloads.randn_bf16((1, tot, Hkv, 128), 13)
    out = gqa.gqa_attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=causal,
                               cu_seqlens=to_dev(cu), max_seqlen=max(lens))
    torch.cuda.synchronize()
    ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=causal, cu_seqlens=cu)
    assert_bf16_close(to_f64(out), ref, what=str(case))


def test_bf16_causality_is_exact(gqa):
    """Changing keys/values after position t leaves every output row <= t bit-identical
    (course page, typical errors: attention must not see the future)."""
    say("bf16 causality")
    q = to_dev(workloads.randn_bf16((1, 256, 8, 128), 21))
    k = to_dev(workloads.randn_bf16((1, 256, 2, 128), 22))
    v = to_dev(workloads.randn_bf16((1, 256, 2, 128), 23))
    base = gqa.gqa_attn_prefill(q, k, v, causal=True)
    for t in (0, 63, 64, 130, 254):
        k2, v2 = k.clone(), v.clone()
        k2[:, t + 1:] = k2[:, t + 1:] * 3 + 1
        v2[:, t + 1:] = -v2[:, t + 1:]
        o = gqa.gqa_attn_prefill(q, k2, v2, causal=True)
        assert torch.equal(o[:, :t + 1], base[:, :t + 1]), t


def test_bf16_closed_forms(gqa):
    """V == 1 gives 1 (rows sum to one); K == 0 gives the running mean of V."""
    say("bf16 closed forms")
    q = to_dev(workloads.randn_bf16((1, 200, 8, 128), 31))
    k = to_dev(workloads.randn_bf16((1, 200, 2, 128), 32))
    ones = torch.ones(1, 200, 2, 128, dtype=torch.bfloat16, device="cuda")
    o = gqa.gqa_attn_prefill(q, k, ones, causal=True).float()
    assert torch.max(torch.abs(o - 1)).item() <= 2 ** -8
    v = workloads.randn_bf16((1, 200, 2, 128), 33)
    z = torch.zeros(1, 200, 2, 128, dtype=torch.bfloat16, device="cuda")
    o = gqa.gqa_attn_prefill(q, z, to_dev(v), causal=True).double().cpu()
    vf = v.double()
    mean = torch.cumsum(vf, dim=1) / torch.arange(1, 201, dtype=torch.float64)[None, :, None, None]
    want = mean.repeat_interleave(4, dim=2)
    err = torch.max(torch.abs(o - want)).item()
    assert err <= 2e-2 and err / torch.max(torch.abs(want)).item() <= 1e-2, err


def test_bf16_deterministic(gqa):
    say("bf16 determinism")
    q = to_dev(workloads.randn_bf16((2, 333, 32, 128), 41))
    k = to_dev(workloads.randn_bf16((2, 333, 8, 128), 42))
    v = to_dev(workloads.randn_bf16((2, 333, 8, 128), 43))
    a = gqa.gqa_attn_prefill(q, k, v, causal=True)
    b = gqa.gqa_attn_prefill(q, k, v, causal=True)
    assert torch.equal(a, b)


# ------------------------------------------------------------------------------------------------
# decode (split-KV + combine)
# ------------------------------------------------------------------------------------------------

DECODE_CASES = [
    # B, Tkv, Hq, Hkv, d
    (3, 1000, 8, 2, 128),
    (2, 77, 32, 1, 64),
    (5, 4096, 32, 8, 128),
    (4, 300, 12, 4, 128),   # G = 3
    (1, 1, 4, 2, 128),      # a single cached key
    (2, 33, 16, 1, 128),    # G = 16: every head column used; one key past a tile
    (1, 5000, 40, 2, 128),  # G = 20: a second, partial chunk of query heads
    (3, 31, 4, 1, 64),      # shorter than one key tile
    (2, 8192, 8, 8, 64),    # G = 1 (multi-head)
    (2, 300, 64, 1, 128),   # G = 64: two workgroups of two 16-head chunks per sequence
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "B{}_Tkv{}_Hq{}_Hkv{}_d{}".format(*c))
def test_bf16_decode_vs_oracle(gqa, orc, case):
    B, Tkv, Hq, Hkv, d = case
    say(f"bf16 decode {case}")
    q = workloads.randn_bf16((B, 1, Hq, d), 51)
    k = workloads.randn_bf16((B, Tkv, Hkv, d), 52)
    v = workloads.randn_bf16((B, Tkv, Hkv, d), 53)
    out = gqa.gqa_attn_decode(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=True)
    assert_bf16_close(to_f64(out), ref, what=str(case))


def test_bf16_decode_growing_logits(gqa, orc):
    """Key norms grow along the cache, so the running maximum keeps rising from tile to tile and
    the softmax reference is moved many times; the result must still match the two-pass oracle."""
    say("bf16 decode growing logits")
    B, Tkv, Hq, Hkv, d = 2, 3000, 8, 2, 128
    q = workloads.randn_bf16((B, 1, Hq, d), 54)
    ramp = 0.2 + 4.0 * torch.arange(Tkv, dtype=torch.float32).reshape(1, Tkv, 1, 1) / Tkv
    k = workloads.to_bf16(workloads.randn_f32((B, Tkv, Hkv, d), 55) * ramp)
    v = workloads.randn_bf16((B, Tkv, Hkv, d), 56)
    out = gqa.gqa_attn_decode(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=True)
    assert_bf16_close(to_f64(out), ref, what="growing logits")


def test_f32_decode_vs_oracle(gqa, orc):
    say("f32 decode")
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 1, 8, 16)).astype(np.float32)
    k = rng.standard_normal((3, 100, 2, 16)).astype(np.float32)
    v = rng.standard_normal((3, 100, 2, 16)).astype(np.float32)
    out = gqa.gqa_attn_decode(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    assert_f32_close(to_f64(out), orc.attention(q, k, v))


def test_decode_matches_prefill_row(gqa):
    say("decode vs prefill one row")
    q = to_dev(workloads.randn_bf16((4, 1, 32, 128), 61))
    k = to_dev(workloads.randn_bf16((4, 2000, 8, 128), 62))
    v = to_dev(workloads.randn_bf16((4, 2000, 8, 128), 63))
    a = gqa.gqa_attn_decode(q, k, v).float()
    b = gqa.gqa_attn_prefill(q, k, v, causal=True).float()
    assert torch.max(torch.abs(a - b)).item() <= 2 ** -7 * torch.max(torch.abs(b)).item()


# ------------------------------------------------------------------------------------------------
# fold (bf16)
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("g", [8, 4, 2, 1])
def test_bf16_fold_vs_oracle(gqa, orc, g):
    say(f"bf16 fold g={g}")
    x = workloads.randn_bf16((2, 37, 8, 128), 71)
    y = gqa.gqa_fold_kv(to_dev(x), g)
    torch.cuda.synchronize()
    ref = orc.fold_kv(host_view(x), g)
    got = to_f64(y)
    # one rounding of the fp32 mean to bf16: within one bf16 ulp (2^-8 relative) of the mean
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    if g == 8:
        assert torch.equal(y.cpu(), x)
