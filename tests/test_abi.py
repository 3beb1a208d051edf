"""The C-ABI library on the CPU: it loads, exports every function the header declares, and its
argument validation returns the documented status codes before any HIP call is made (every
call here fails validation, so nothing is enqueued and no GPU is needed)."""
import ctypes
import os

import pytest

import grouped_query_softmax_amd as gqa
from grouped_query_softmax_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return gqa.raw_library()


def test_library_exports_every_header_function(lib):
    names = gqa.header_functions()
    assert set(names) >= {"gqa_attn_prefill", "gqa_attn_decode", "gqa_attn_decode_workspace_bytes",
                          "gqa_fold_kv", "gqa_status_string", "gqa_attn_abi_version"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.gqa_attn_abi_version() == 3


# The boundary's core calls as the interface specification writes them (whitespace aside).
SPEC_PROTOTYPES = [
    "gqa_status_t gqa_attn_prefill(const void* q, const void* k, const void* v, void* out, int B, "
    "int Tq, int Tkv, int Hq, int Hkv, int d, float scale, int causal, "
    "const int32_t* cu_seqlens, int max_seqlen, gqa_dtype_t dtype, hipStream_t stream);",
    "size_t gqa_attn_decode_workspace_bytes(int B, int Tkv, int Hq, int d);",
    "gqa_status_t gqa_attn_decode(const void* q, const void* k_cache, const void* v_cache, "
    "void* out, int B, int Tkv, int Hq, int Hkv, int d, float scale, int causal, "
    "void* workspace, size_t workspace_bytes, gqa_dtype_t dtype, hipStream_t stream);",
    "gqa_status_t gqa_fold_kv(const void* src, void* dst, int B, int T, int H, int g, int d, "
    "gqa_dtype_t dtype, hipStream_t stream);",
    "const char* gqa_status_string(gqa_status_t s);",
]


def _norm_ws(text):
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    return re.sub(r"\s+", " ", text).replace("( ", "(").replace(" )", ")")


def test_header_declares_the_specified_signatures_and_codes():
    text = _norm_ws(open(os.path.join(ROOT, "include", "gqa_attn.h")).read())
    for proto in SPEC_PROTOTYPES:
        assert _norm_ws(proto) in text, proto
    codes = {"GQA_OK": 0, "GQA_ERR_NULL_PTR": 1, "GQA_ERR_SHAPE": 2, "GQA_ERR_GROUPING": 3,
             "GQA_ERR_UNSUPPORTED": 4, "GQA_ERR_WORKSPACE": 5, "GQA_ERR_HIP": 6}
    for name, value in codes.items():
        assert f"{name} = {value}" in text, name
        assert getattr(B, name) == value
    assert "GQA_DTYPE_F32 = 0" in text and "GQA_DTYPE_BF16 = 1" in text
    assert B.GQA_ERR_ALIAS == 7 and "GQA_ERR_ALIAS = 7" in text


def test_decode_workspace_bound_covers_every_grouping(lib):
    for (Bn, Tkv, Hq, d) in [(64, 8192, 32, 128), (1, 131072, 32, 128), (3, 1000, 40, 64),
                             (5, 300, 7, 128)]:
        bound = lib.gqa_attn_decode_workspace_bytes(Bn, Tkv, Hq, d)
        exact = [lib.gqa_attn_decode_workspace_bytes_hkv(Bn, Tkv, Hq, h, d)
                 for h in range(1, Hq + 1) if Hq % h == 0]
        assert bound == max(exact) and all(e > 0 for e in exact)
    assert lib.gqa_attn_decode_workspace_bytes(0, 8, 8, 128) == 0
    assert lib.gqa_attn_decode_workspace_bytes(1, 8, 8, -1) == 0


def test_scale_default_and_invalid(lib):
    # GQA_SCALE_DEFAULT passes validation (a later check fails instead); a negative or infinite
    # scale is a shape error
    assert pre(lib, scale=B.GQA_SCALE_DEFAULT, o=Q + 64) == B.GQA_ERR_ALIAS
    assert pre(lib, scale=-0.1) == B.GQA_ERR_SHAPE
    assert pre(lib, scale=float("inf")) == B.GQA_ERR_SHAPE


def test_single_hip_runtime_in_process():
    assert len(B._hip_runtimes_mapped()) <= 1


def test_status_strings(lib):
    for code in range(8):
        s = gqa.gqa_status_string(code)
        assert s and s != "unknown status"
    assert gqa.gqa_status_string(99) == "unknown status"


# fake, 16-byte aligned, non-overlapping addresses; validation never dereferences them
Q, K, V, O, W = (0x10000000 * i for i in (1, 2, 3, 4, 5))
F32, BF16 = B.GQA_DTYPE_F32, B.GQA_DTYPE_BF16


def pre(lib, q=Q, k=K, v=V, o=O, Bn=1, Tq=8, Tkv=8, Hq=8, Hkv=2, d=128, scale=0.1, causal=0,
        cu=None, msl=0, dt=BF16):
    return lib.gqa_attn_prefill(q, k, v, o, Bn, Tq, Tkv, Hq, Hkv, d, scale, causal, cu, msl, dt,
                                None)


def test_prefill_validation(lib):
    assert pre(lib, q=None) == B.GQA_ERR_NULL_PTR
    assert pre(lib, o=None) == B.GQA_ERR_NULL_PTR
    assert pre(lib, Tq=0) == B.GQA_ERR_SHAPE
    assert pre(lib, Hkv=-1) == B.GQA_ERR_SHAPE
    assert pre(lib, Hq=8, Hkv=3) == B.GQA_ERR_GROUPING
    assert pre(lib, d=96) == B.GQA_ERR_UNSUPPORTED
    assert pre(lib, d=16) == B.GQA_ERR_UNSUPPORTED          # bf16 needs 64 or 128
    assert pre(lib, dt=7) == B.GQA_ERR_UNSUPPORTED
    assert pre(lib, q=Q + 8) == B.GQA_ERR_UNSUPPORTED       # misaligned
    assert pre(lib, Tq=9, Tkv=8, causal=1) == B.GQA_ERR_SHAPE
    assert pre(lib, scale=float("nan")) == B.GQA_ERR_SHAPE
    assert pre(lib, o=Q + 64) == B.GQA_ERR_ALIAS             # out overlaps q
    assert pre(lib, o=K) == B.GQA_ERR_ALIAS
    # packed batch: Tq must equal Tkv, max_seqlen in (0, Tq]
    assert pre(lib, cu=W, msl=0) == B.GQA_ERR_SHAPE
    assert pre(lib, cu=W, Tq=8, Tkv=9, msl=4) == B.GQA_ERR_SHAPE
    assert pre(lib, cu=W, msl=9) == B.GQA_ERR_SHAPE
    # launch limits: f32 runs a 3-D grid (at most 65535 items); bf16 addresses one item's keys
    # and values with 32-bit offsets (at most 2 GiB per item)
    assert pre(lib, Bn=70000, d=16, dt=F32) == B.GQA_ERR_UNSUPPORTED
    assert pre(lib, Tkv=1 << 22, Hq=8, Hkv=8) == B.GQA_ERR_UNSUPPORTED


def test_window_and_ragged_validation(lib):
    def prew(window=4, n_sink=0, dt=BF16, d=128):
        return lib.gqa_attn_prefill_window(Q, K, V, O, 1, 8, 8, 8, 2, d, 0.1, window, n_sink,
                                           None, 0, dt, None)
    assert prew(window=-1) == B.GQA_ERR_SHAPE
    assert prew(n_sink=-2) == B.GQA_ERR_SHAPE
    assert prew(dt=F32, d=16) == B.GQA_ERR_UNSUPPORTED     # windows are bf16 only
    assert lib.gqa_attn_prefill_window(Q, K, V, O, 1, 9, 8, 8, 2, 128, 0.1, 4, 0, None, 0, BF16,
                                       None) == B.GQA_ERR_SHAPE   # causal needs Tq <= Tkv
    need = lib.gqa_attn_decode_workspace_bytes_hkv(4, 1024, 32, 8, 128)

    def rag(window=0, n_sink=0, dt=BF16, d=128, lens=W + 4096, ws=W, wsb=need, Tmax=1024):
        return lib.gqa_attn_decode_ragged(Q, K, V, O, 4, Tmax, 32, 8, d, 0.1, lens, window,
                                          n_sink, ws, wsb, dt, None)
    assert rag(window=-3) == B.GQA_ERR_SHAPE
    assert rag(n_sink=-1) == B.GQA_ERR_SHAPE
    assert rag(dt=F32, d=16) == B.GQA_ERR_UNSUPPORTED
    assert rag(ws=None) == B.GQA_ERR_WORKSPACE
    assert rag(Tmax=1 << 22) == B.GQA_ERR_UNSUPPORTED


def test_window_cache_validation(lib):
    Opt = B.AttnOptions
    need = lib.gqa_attn_decode_workspace_bytes_hkv(4, 68, 32, 8, 128)

    def wc(window=64, n_sink=4, dt=BF16, d=128, lens=W + 4096, opt=True, ws=W, wsb=need, hkv=8):
        o = Opt(window, n_sink, None, None, 0, None, None, None, 0.0, 0)
        return lib.gqa_attn_decode_window_cache(Q, K, V, O, 4, 32, hkv, d, 0.1, lens,
                                                ctypes.byref(o) if opt else None, ws, wsb, dt,
                                                None)
    assert wc(lens=None) == B.GQA_ERR_NULL_PTR            # the entry counts are required
    assert wc(opt=False) == B.GQA_ERR_NULL_PTR            # so is the window
    assert wc(window=0) == B.GQA_ERR_SHAPE
    assert wc(n_sink=-1) == B.GQA_ERR_SHAPE
    assert wc(window=2**31 - 1) == B.GQA_ERR_SHAPE        # n_sink + window past int
    assert wc(dt=F32, d=16) == B.GQA_ERR_UNSUPPORTED
    assert wc(hkv=5) == B.GQA_ERR_GROUPING
    assert wc(wsb=need - 1) == B.GQA_ERR_WORKSPACE        # sized for n_sink + window slots


def test_extended_options_validation(lib):
    Opt = B.AttnOptions
    T = W + 8192   # fake 16-byte aligned table addresses

    def pex(opt, causal=1, dt=BF16, d=128, Tkv=8):
        return lib.gqa_attn_prefill_ex(Q, K, V, O, 1, 8, Tkv, 8, 2, d, 0.1, causal, None, 0,
                                       ctypes.byref(opt) if opt is not None else None, dt, None)
    assert pex(Opt(0, 0, T, None, 8, None)) == B.GQA_ERR_NULL_PTR    # one table missing
    assert pex(Opt(0, 0, T, T + 4096, 7, None)) == B.GQA_ERR_SHAPE         # fewer rows than keys
    assert pex(Opt(0, 0, T + 4, T + 4096, 8, None)) == B.GQA_ERR_UNSUPPORTED  # misaligned table
    assert pex(Opt(0, 0, T, T + 4096, 8, None), dt=F32, d=16) == B.GQA_ERR_UNSUPPORTED
    assert pex(Opt(3, 0, None, None, 0, None), causal=0) == B.GQA_ERR_SHAPE  # windows are causal
    assert pex(Opt(-1, 0, None, None, 0, None)) == B.GQA_ERR_SHAPE
    need = lib.gqa_attn_decode_workspace_bytes_hkv(4, 1024, 32, 8, 128)

    def dex(opt, Tmax=1024):
        return lib.gqa_attn_decode_ex(Q, K, V, O, 4, Tmax, 32, 8, 128, 0.1, None,
                                      ctypes.byref(opt), W, need, BF16, None)
    assert dex(Opt(0, 0, T, T + 4096, 1023, None)) == B.GQA_ERR_SHAPE      # rows must cover Tmax
    assert dex(Opt(0, 0, None, T, 1024, None)) == B.GQA_ERR_NULL_PTR


def test_qk_norm_options_validation(lib):
    Opt = B.AttnOptions
    N = W + 65536   # fake aligned weight addresses

    def pex(opt, dt=BF16, d=128):
        return lib.gqa_attn_prefill_ex(Q, K, V, O, 1, 8, 8, 8, 2, d, 0.1, 1, None, 0,
                                       ctypes.byref(opt), dt, None)
    assert pex(Opt(0, 0, None, None, 0, None, N, None, 1e-6)) == B.GQA_ERR_NULL_PTR
    assert pex(Opt(0, 0, None, None, 0, None, N, N + 4096, 0.0)) == B.GQA_ERR_SHAPE
    assert pex(Opt(0, 0, None, None, 0, None, N, N + 4096, float("nan"))) == B.GQA_ERR_SHAPE
    assert pex(Opt(0, 0, None, None, 0, None, N + 4, N + 4096, 1e-6)) == B.GQA_ERR_UNSUPPORTED
    assert pex(Opt(0, 0, None, None, 0, None, N, N + 4096, 1e-6), dt=F32, d=16) == \
        B.GQA_ERR_UNSUPPORTED


def test_prepare_keys_validation(lib):
    Opt = B.AttnOptions
    N, T = W + 65536, W + 8192

    def prep(opt, k=K, out=O, dt=BF16, d=128, pos0=0, Tn=8):
        return lib.gqa_prepare_keys(k, out, 2, Tn, 2, d, None, 0, pos0,
                                    ctypes.byref(opt) if opt is not None else None, dt, None)
    ok_norm = Opt(0, 0, None, None, 0, None, None, N, 1e-6)
    assert prep(None) == B.GQA_ERR_NULL_PTR
    assert prep(Opt()) == B.GQA_ERR_SHAPE                       # nothing to apply
    assert prep(ok_norm, dt=F32, d=16) == B.GQA_ERR_UNSUPPORTED
    assert prep(Opt(0, 0, T, T + 4096, 8, None), pos0=1) == B.GQA_ERR_SHAPE  # table too short
    assert prep(ok_norm, pos0=-1) == B.GQA_ERR_SHAPE
    assert prep(ok_norm, out=K + 64) == B.GQA_ERR_ALIAS         # partial overlap
    assert prep(Opt(0, 0, None, None, 0, None, None, N, 0.0)) == B.GQA_ERR_SHAPE


def test_gva_validation(lib):
    Opt = B.AttnOptions
    T = W + 8192

    def gva(q=Q, o=O, H=2, HV=8, d=128, dt=BF16, causal=1, Tq=8, Tkv=8, opt=None):
        return lib.gqa_attn_prefill_gva(q, K, V, o, 1, Tq, Tkv, H, HV, d, 0.1, causal, None, 0,
                                        ctypes.byref(opt) if opt is not None else None, dt, None)
    assert gva(q=None) == B.GQA_ERR_NULL_PTR
    assert gva(HV=7) == B.GQA_ERR_GROUPING             # value heads do not group evenly
    assert gva(H=0) == B.GQA_ERR_SHAPE
    assert gva(dt=F32, d=16) == B.GQA_ERR_UNSUPPORTED  # bf16 only
    assert gva(d=96) == B.GQA_ERR_UNSUPPORTED
    assert gva(Tq=9) == B.GQA_ERR_SHAPE                # causal needs Tq <= Tkv
    assert gva(opt=Opt(0, 0, T, T + 4096, 8, None)) == B.GQA_ERR_UNSUPPORTED  # no rotary here
    assert gva(causal=0, opt=Opt(4, 0, None, None, 0, None)) == B.GQA_ERR_SHAPE  # window: causal
    assert gva(o=V + 64) == B.GQA_ERR_ALIAS            # output over the values


def test_backward_validation(lib):
    need = lib.gqa_attn_backward_workspace_bytes(2, 8, 8)
    assert need >= 2 * 8 * 8 * 4 and need % 16 == 0
    X = 0x100000000  # more fake, aligned, non-overlapping addresses
    L, DQ, DK, DV, DO = (X + 0x10000000 * i for i in range(5))

    def bwd(q=Q, lse=L, dq=DQ, ws=W, wsb=need, dt=BF16, d=128, causal=0, Tq=8, Tkv=8, Hkv=2):
        return lib.gqa_attn_backward(q, K, V, O, DO, lse, dq, DK, DV, 2, Tq, Tkv, 8, Hkv, d, 0.1,
                                     causal, ws, wsb, dt, None)
    assert bwd(lse=None) == B.GQA_ERR_NULL_PTR
    assert bwd(Hkv=3) == B.GQA_ERR_GROUPING
    assert bwd(dt=F32, d=16) == B.GQA_ERR_UNSUPPORTED
    assert bwd(Tq=9, causal=1) == B.GQA_ERR_SHAPE
    assert bwd(ws=None) == B.GQA_ERR_WORKSPACE
    assert bwd(wsb=need - 16) == B.GQA_ERR_WORKSPACE
    assert bwd(dq=Q) == B.GQA_ERR_ALIAS             # gradient over its input
    assert bwd(ws=DQ) == B.GQA_ERR_ALIAS            # workspace over a gradient


def test_decode_validation(lib):
    need = lib.gqa_attn_decode_workspace_bytes_hkv(4, 1024, 32, 8, 128)
    assert need > 0 and need % 16 == 0
    assert lib.gqa_attn_decode_workspace_bytes_hkv(4, 1024, 32, 5, 128) == 0

    def dec(q=Q, k=K, v=V, o=O, Bn=4, Tkv=1024, Hq=32, Hkv=8, d=128, ws=W, wsb=need, dt=BF16):
        return lib.gqa_attn_decode(q, k, v, o, Bn, Tkv, Hq, Hkv, d, 0.1, 0, ws, wsb, dt, None)

    assert dec(k=None) == B.GQA_ERR_NULL_PTR
    assert dec(Tkv=0) == B.GQA_ERR_SHAPE
    assert dec(Hkv=5) == B.GQA_ERR_GROUPING
    assert dec(d=80) == B.GQA_ERR_UNSUPPORTED
    assert dec(ws=None) == B.GQA_ERR_WORKSPACE
    assert dec(wsb=need - 1) == B.GQA_ERR_WORKSPACE
    assert dec(ws=W + 4) == B.GQA_ERR_UNSUPPORTED
    assert dec(o=Q) == B.GQA_ERR_ALIAS
    assert dec(ws=O) == B.GQA_ERR_ALIAS
    # one sequence's cache beyond 2 GiB (32-bit offsets) is refused before anything else
    assert dec(Tkv=1 << 22) == B.GQA_ERR_UNSUPPORTED


def test_fold_validation(lib):
    def fold(s=Q, dst=O, Bn=1, T=4, H=8, g=2, d=16, dt=F32):
        return lib.gqa_fold_kv(s, dst, Bn, T, H, g, d, dt, None)

    assert fold(s=None) == B.GQA_ERR_NULL_PTR
    assert fold(g=0) == B.GQA_ERR_SHAPE
    assert fold(g=3) == B.GQA_ERR_GROUPING
    assert fold(d=6) == B.GQA_ERR_UNSUPPORTED       # rows must be whole 16-byte vectors
    assert fold(dst=Q + 16) == B.GQA_ERR_ALIAS


def test_python_wrapper_raises_value_error_for_uneven_heads():
    import torch
    with pytest.raises(gqa.GQAValueError) as e:
        gqa.gqa_fold_kv(torch.empty(1, 2, 8, 16), 3)
    assert e.value.code == B.GQA_ERR_GROUPING


def test_header_cites_and_documents_each_entry_point():
    text = open(os.path.join(ROOT, "include", "gqa_attn.h")).read()
    for n in ("gqa_attn_prefill", "gqa_attn_decode", "gqa_fold_kv"):
        assert n in text
    assert "GQA lab page" in text and "Week 7. Attention" in text
