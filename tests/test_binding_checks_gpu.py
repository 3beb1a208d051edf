"""The Python binding refuses mis-shaped arguments before anything is enqueued: every call here
raises on the host (the tensors live on the device because the binding accepts nothing else)."""
import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gqa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_query_softmax_amd as g
    return g


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def test_decode_rejects_bad_out(gqa):
    say("binding: decode out checks")
    q, k = _t(2, 1, 8, 128), _t(2, 64, 2, 128)
    for bad in (_t(2, 1, 4, 128), _t(2, 1, 8, 128, dtype=torch.float32),
                _t(2, 1, 8, 256)[..., :128]):
        assert bad.shape != q.shape or bad.dtype != q.dtype or not bad.is_contiguous()
        with pytest.raises(ValueError):
            gqa.gqa_attn_decode(q, k, k, out=bad)
        with pytest.raises(ValueError):
            gqa.gqa_attn_decode_ragged(q, k, k, out=bad)
        with pytest.raises(ValueError):
            gqa.gqa_attn_decode_ex(q, k, k, out=bad)


def test_fold_rejects_bad_out(gqa):
    say("binding: fold out checks")
    src = _t(1, 4, 8, 64)
    for bad in (_t(1, 4, 4, 64), _t(1, 4, 2, 64, dtype=torch.float32),
                _t(1, 2, 4, 64).transpose(1, 2)):
        assert bad.shape != (1, 4, 2, 64) or bad.dtype != src.dtype or not bad.is_contiguous()
        with pytest.raises(ValueError):
            gqa.gqa_fold_kv(src, 2, out=bad)


def test_backward_rejects_mismatched_keys(gqa):
    say("binding: backward shape checks")
    q = _t(2, 16, 8, 128)
    lse = _t(2, 16, 8, dtype=torch.float32)
    for k in (_t(1, 16, 2, 128), _t(2, 16, 2, 64)):
        with pytest.raises(ValueError):
            gqa.gqa_attn_backward(q, k, k, q, q, lse)


def test_packed_prefill_needs_max_seqlen(gqa):
    say("binding: packed calls need max_seqlen")
    q, k = _t(1, 24, 8, 128), _t(1, 24, 2, 128)
    cu = torch.tensor([0, 10, 24], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        gqa.gqa_attn_prefill(q, k, k, causal=True, cu_seqlens=cu)
    with pytest.raises(ValueError):
        gqa.gqa_attn_prefill_window(q, k, k, window=4, cu_seqlens=cu)
    with pytest.raises(ValueError):
        gqa.gqa_prepare_keys(k, qk_norm=(None, _t(128, dtype=torch.float32), 1e-6),
                             cu_seqlens=cu)


def test_window_cache_decode_rejects_bad_arguments(gqa):
    say("binding: bounded-cache decode checks")
    q, ring = _t(2, 1, 8, 128), _t(2, 68, 2, 128)   # 4 sinks + a window of 64 slots
    lens = torch.tensor([5, 500], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):   # the cache must hold n_sink + window slots
        gqa.gqa_attn_decode_window_cache(q, ring, ring, lens, window=64, n_sink=5)
    with pytest.raises(ValueError):
        gqa.gqa_attn_decode_window_cache(q, ring, ring, lens, window=0, n_sink=68)
    with pytest.raises(ValueError):
        gqa.gqa_attn_decode_window_cache(q, ring, ring, lens, window=64, n_sink=-1)
    for bad in (lens[:1], lens.to(torch.int64), lens.cpu()):
        with pytest.raises((ValueError, TypeError)):
            gqa.gqa_attn_decode_window_cache(q, ring, ring, bad, window=64, n_sink=4)
    with pytest.raises(ValueError):
        gqa.gqa_attn_decode_window_cache(q, ring, ring, lens, window=64, n_sink=4,
                                         out=_t(2, 1, 4, 128))
