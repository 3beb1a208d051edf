"""The allocation-free decode entry point, through the C ABI: its output equals gqa_attn_decode's
(with a caller workspace) bit for bit, on two calls in a row, the second one smaller (the
library's scratch keeps the first call's partials, which must not leak into the second)."""
import ctypes

import pytest
import torch

import workloads
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gqa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_query_softmax_amd as g
    return g


def _decode_both(gqa, B, Tkv, Hq, Hkv, d, seed):
    lib = gqa.raw_library()
    q = to_dev(workloads.randn_bf16((B, 1, Hq, d), seed))
    k = to_dev(workloads.randn_bf16((B, Tkv, Hkv, d), seed + 1))
    v = to_dev(workloads.randn_bf16((B, Tkv, Hkv, d), seed + 2))
    stream = torch.cuda.current_stream().cuda_stream
    need = lib.gqa_attn_decode_workspace_bytes_hkv(B, Tkv, Hq, Hkv, d)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    ref = torch.empty_like(q)
    rc = lib.gqa_attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), ref.data_ptr(), B, Tkv,
                             Hq, Hkv, d, ctypes.c_float(0.0), 0, ws.data_ptr(), ws.numel(), 1,
                             ctypes.c_void_p(stream))
    assert rc == 0, rc
    got = torch.full_like(q, float("nan"))
    rc = lib.gqa_attn_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), got.data_ptr(), B,
                                     Tkv, Hq, Hkv, d, ctypes.c_float(0.0), 0, 1,
                                     ctypes.c_void_p(stream))
    assert rc == 0, rc
    torch.cuda.synchronize()
    return ref, got


# (first call, second smaller call): several splits per sequence in both, so the scratch is used
CASES = [((2, 8192, 32, 8, 128), (1, 3000, 32, 8, 128)),
         ((3, 5000, 40, 2, 128), (2, 700, 16, 4, 64))]


@pytest.mark.parametrize("pair", CASES, ids=lambda p: f"{p[0]}->{p[1]}")
def test_noalloc_decode_matches_workspace_decode(gqa, pair):
    for i, (B, Tkv, Hq, Hkv, d) in enumerate(pair):
        say(f"no-alloc decode call {i}: B={B} Tkv={Tkv} Hq={Hq} Hkv={Hkv} d={d}")
        lib = gqa.raw_library()
        assert lib.gqa_attn_decode_workspace_bytes_hkv(B, Tkv, Hq, Hkv, d) > B * Hq * (d + 2) * 4
        ref, got = _decode_both(gqa, B, Tkv, Hq, Hkv, d, 300 + 10 * i)
        assert torch.equal(ref, got), (i, (ref.float() - got.float()).abs().max().item())


def test_noalloc_decode_refuses_oversized(gqa):
    """1024 sequences x 32 query heads: the partials (one split each) exceed the fixed scratch, so
    the call is refused before anything is enqueued (the buffers are real and valid)."""
    say("no-alloc decode: oversized request")
    lib = gqa.raw_library()
    B, Tkv, Hq, Hkv, d = 1024, 1, 32, 8, 128
    assert lib.gqa_attn_decode_workspace_bytes_hkv(B, Tkv, Hq, Hkv, d) > \
        gqa.GQA_DECODE_SCRATCH_BYTES
    q = torch.zeros((B, 1, Hq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Tkv, Hkv, d), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(q)
    rc = lib.gqa_attn_decode_noalloc(q.data_ptr(), k.data_ptr(), k.data_ptr(), out.data_ptr(), B,
                                     Tkv, Hq, Hkv, d, ctypes.c_float(0.0), 0, 1, None)
    assert rc == 5  # GQA_ERR_WORKSPACE
    with pytest.raises(RuntimeError):
        gqa.gqa_attn_decode_noalloc(q, k, k, out=out)


def test_noalloc_binding_matches(gqa):
    say("no-alloc decode through the binding")
    q = to_dev(workloads.randn_bf16((4, 1, 32, 128), 401))
    k = to_dev(workloads.randn_bf16((4, 4096, 8, 128), 402))
    v = to_dev(workloads.randn_bf16((4, 4096, 8, 128), 403))
    a = gqa.gqa_attn_decode(q, k, v)
    b = gqa.gqa_attn_decode_noalloc(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
