"""ctypes binding of ``libgqa_attn.so`` (argument marshalling only).

Every step of the attention runs in the library's HIP kernels; this module only checks that the
library is present, turns torch tensors into pointers, sizes and a stream handle, and maps status
codes to Python exceptions (ValueError for sizes and uneven head groups, like the GQA lab page's
ValueError convention; RuntimeError otherwise). There is no fallback: if the library is missing,
importing this module fails.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch  # loaded first so the library binds to the HIP runtime torch already mapped

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgqa_attn.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "gqa_attn.h")

GQA_OK, GQA_ERR_NULL_PTR, GQA_ERR_SHAPE, GQA_ERR_GROUPING = 0, 1, 2, 3
GQA_ERR_UNSUPPORTED, GQA_ERR_WORKSPACE, GQA_ERR_HIP, GQA_ERR_ALIAS = 4, 5, 6, 7
GQA_DTYPE_F32, GQA_DTYPE_BF16 = 0, 1
# scale argument that makes the library use 1/sqrt(d)
GQA_SCALE_DEFAULT = 0.0
# size of the library's per-GPU decode scratch (gqa_attn_decode_noalloc)
GQA_DECODE_SCRATCH_BYTES = 16 << 20


class GQAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


class GQAValueError(ValueError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln and "/" in ln})
    except OSError:
        return []


class AttnOptions(ctypes.Structure):
    """``gqa_attn_options_t``: sliding window, sinks, rotary tables, log-sum-exp output and
    QK-norm weights of the extended calls."""
    _fields_ = [("window", ctypes.c_int), ("n_sink", ctypes.c_int),
                ("rope_cos", ctypes.c_void_p), ("rope_sin", ctypes.c_void_p),
                ("rope_rows", ctypes.c_int), ("lse", ctypes.c_void_p),
                ("q_norm_w", ctypes.c_void_p), ("k_norm_w", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float), ("keys_prepared", ctypes.c_int)]


def _options(window: int, n_sink: int, rope, d: int, lse=None, qk_norm=None,
             keys_prepared: bool = False) -> AttnOptions:
    """qk_norm: None or (w_q, w_k, eps), float32 device weights [d]. The returned struct keeps
    the tensors it points to alive (``_keep``) until the call has been enqueued."""
    o = AttnOptions(int(window), int(n_sink), None, None, 0, None, None, None, 0.0,
                    int(bool(keys_prepared)))
    keep = []
    if lse is not None:
        o.lse = lse.data_ptr()
    if rope is not None:
        cos_t, sin_t = (_dev(t, name) for t, name in zip(rope, ("rope cos", "rope sin")))
        if (cos_t.dtype != torch.float32 or sin_t.dtype != torch.float32 or cos_t.dim() != 2
                or cos_t.shape != sin_t.shape or cos_t.shape[1] * 2 != d):
            raise ValueError("rope tables must be float32 device tensors [rows, d/2]")
        o.rope_cos, o.rope_sin, o.rope_rows = cos_t.data_ptr(), sin_t.data_ptr(), cos_t.shape[0]
        keep += [cos_t, sin_t]
    if qk_norm is not None:
        ws = [None if t is None else _dev(t, name)
              for t, name in zip(qk_norm[:2], ("q norm weights", "k norm weights"))]
        for t in ws:
            if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (d,)):
                raise ValueError("qk-norm weights must be float32 device tensors [d]")
        o.q_norm_w = ws[0].data_ptr() if ws[0] is not None else None
        o.k_norm_w = ws[1].data_ptr() if ws[1] is not None else None
        o.norm_eps = float(qk_norm[2])
        keep += [t for t in ws if t is not None]
    o._keep = keep
    return o


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python grouped_query_softmax_amd/build.py`")
    lib = ctypes.CDLL(path)
    P, I, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.gqa_attn_prefill.argtypes = [P, P, P, P, I, I, I, I, I, I, F, I, P, I, I, P]
    lib.gqa_attn_prefill.restype = I
    lib.gqa_attn_decode_workspace_bytes.argtypes = [I, I, I, I]
    lib.gqa_attn_decode_workspace_bytes.restype = SZ
    lib.gqa_attn_decode_workspace_bytes_hkv.argtypes = [I, I, I, I, I]
    lib.gqa_attn_decode_workspace_bytes_hkv.restype = SZ
    lib.gqa_attn_decode.argtypes = [P, P, P, P, I, I, I, I, I, F, I, P, SZ, I, P]
    lib.gqa_attn_decode.restype = I
    lib.gqa_attn_decode_noalloc.argtypes = [P, P, P, P, I, I, I, I, I, F, I, I, P]
    lib.gqa_attn_decode_noalloc.restype = I
    lib.gqa_attn_prefill_window.argtypes = [P, P, P, P, I, I, I, I, I, I, F, I, I, P, I, I, P]
    lib.gqa_attn_prefill_window.restype = I
    lib.gqa_attn_decode_ragged.argtypes = [P, P, P, P, I, I, I, I, I, F, P, I, I, P, SZ, I, P]
    lib.gqa_attn_decode_ragged.restype = I
    OP = ctypes.POINTER(AttnOptions)
    lib.gqa_attn_prefill_ex.argtypes = [P, P, P, P, I, I, I, I, I, I, F, I, P, I, OP, I, P]
    lib.gqa_attn_prefill_ex.restype = I
    lib.gqa_attn_prefill_gva.argtypes = [P, P, P, P, I, I, I, I, I, I, F, I, P, I, OP, I, P]
    lib.gqa_attn_prefill_gva.restype = I
    lib.gqa_prepare_keys.argtypes = [P, P, I, I, I, I, P, I, I, OP, I, P]
    lib.gqa_prepare_keys.restype = I
    lib.gqa_attn_decode_ex.argtypes = [P, P, P, P, I, I, I, I, I, F, P, OP, P, SZ, I, P]
    lib.gqa_attn_decode_ex.restype = I
    lib.gqa_attn_decode_window_cache.argtypes = [P, P, P, P, I, I, I, I, F, P, OP, P, SZ, I,
                                                 P]
    lib.gqa_attn_decode_window_cache.restype = I
    lib.gqa_attn_backward_workspace_bytes.argtypes = [I, I, I]
    lib.gqa_attn_backward_workspace_bytes.restype = SZ
    lib.gqa_attn_backward.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, SZ, I,
                                      P]
    lib.gqa_attn_backward.restype = I
    lib.gqa_attn_backward_ex.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, I,
                                         OP, P, SZ, I, P]
    lib.gqa_attn_backward_ex.restype = I
    lib.gqa_fold_kv.argtypes = [P, P, I, I, I, I, I, I, P]
    lib.gqa_fold_kv.restype = I
    lib.gqa_status_string.argtypes = [I]
    lib.gqa_status_string.restype = ctypes.c_char_p
    lib.gqa_attn_abi_version.argtypes = []
    lib.gqa_attn_abi_version.restype = I
    return lib


def header_functions(header: str = HEADER):
    """Names of the functions ``include/gqa_attn.h`` declares."""
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", src)))


_lib = load_library()
_runtimes = _hip_runtimes_mapped()
if len(_runtimes) > 1:
    raise ImportError(f"more than one HIP runtime mapped into this process: {_runtimes}")

ABI_VERSION = _lib.gqa_attn_abi_version()


def gqa_status_string(code: int) -> str:
    return _lib.gqa_status_string(code).decode()


def _check(code: int, what: str):
    if code == GQA_OK:
        return
    msg = f"{what}: {gqa_status_string(code)} (status {code})"
    if code in (GQA_ERR_SHAPE, GQA_ERR_GROUPING):
        raise GQAValueError(code, msg)
    raise GQAError(code, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GQA_DTYPE_BF16
    if t.dtype == torch.float32:
        return GQA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    return t if t.is_contiguous() else t.contiguous()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _max_seqlen(max_seqlen) -> int:
    """The longest packed sequence, from the caller: reading it from the device offsets would
    synchronise the stream."""
    if max_seqlen is None:
        raise ValueError("packed batches need max_seqlen (the longest sequence, a host int)")
    return int(max_seqlen)


def _prefill_args(q, k, v, scale, cu_seqlens, max_seqlen, out):
    q, k, v = _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q[B,Tq,Hq,d] and k, v[B,Tkv,Hkv,d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    B, Tq, Hq, d = q.shape
    Bk, Tkv, Hkv, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError("q and k/v disagree on batch or head dim")
    if scale is None:
        scale = GQA_SCALE_DEFAULT
    cu_ptr, nseq, msl = None, B, 0
    if cu_seqlens is not None:
        cu = _dev(cu_seqlens, "cu_seqlens")
        if cu.dtype != torch.int32 or cu.dim() != 1 or cu.numel() < 2:
            raise ValueError("cu_seqlens must be a 1-D int32 device tensor of nseq+1 offsets")
        if B != 1:
            raise ValueError("packed batches use q/k/v of shape [1, total, H, d]")
        nseq = cu.numel() - 1
        cu_ptr, msl = cu.data_ptr(), _max_seqlen(max_seqlen)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    return q, k, v, out, (nseq, Tq, Tkv, Hq, Hkv, d, float(scale)), cu_ptr, msl


def gqa_attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                     scale: Optional[float] = None, cu_seqlens: Optional[torch.Tensor] = None,
                     max_seqlen: Optional[int] = None, out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """q [B,Tq,Hq,d], k/v [B,Tkv,Hkv,d] (or [1,total,H,d] with int32 device cu_seqlens)."""
    q, k, v, out, dims, cu_ptr, msl = _prefill_args(q, k, v, scale, cu_seqlens, max_seqlen, out)
    rc = _lib.gqa_attn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), *dims,
                               int(bool(causal)), cu_ptr, msl, _dtype_code(q), _stream(stream))
    _check(rc, "gqa_attn_prefill")
    return out


def gqa_attn_prefill_window(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, window: int,
                            n_sink: int = 0, scale: Optional[float] = None,
                            cu_seqlens: Optional[torch.Tensor] = None,
                            max_seqlen: Optional[int] = None, out: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """Causal prefill where the query at position p sees keys p-window+1 .. p and the first
    n_sink keys (window 0: plain causal). Shapes as for :func:`gqa_attn_prefill`; bf16 only."""
    q, k, v, out, dims, cu_ptr, msl = _prefill_args(q, k, v, scale, cu_seqlens, max_seqlen, out)
    rc = _lib.gqa_attn_prefill_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      *dims, int(window), int(n_sink), cu_ptr, msl,
                                      _dtype_code(q), _stream(stream))
    _check(rc, "gqa_attn_prefill_window")
    return out


def gqa_attn_prefill_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                        window: int = 0, n_sink: int = 0, rope=None,
                        scale: Optional[float] = None, cu_seqlens: Optional[torch.Tensor] = None,
                        max_seqlen: Optional[int] = None, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, qk_norm=None,
                        keys_prepared: bool = False, stream=None) -> torch.Tensor:
    """:func:`gqa_attn_prefill` with a sliding window / sinks and rotary embedding of q and k
    inside the kernel; rope = (cos, sin) float32 device tables [rows, d/2]; lse: optional float32
    device output [B, Tq, Hq] receiving each row's log-sum-exp (for the backward); qk_norm =
    (w_q, w_k, eps): RMSNorm of every q and k head row before the rotation; keys_prepared: k
    already normalised / turned (:func:`gqa_prepare_keys`), only q is processed. bf16 only."""
    q, k, v, out, dims, cu_ptr, msl = _prefill_args(q, k, v, scale, cu_seqlens, max_seqlen, out)
    if lse is not None:
        lse = _dev(lse, "lse")
        if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(q.shape[:3]) \
                or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 device tensor [B, Tq, Hq]")
    opt = _options(window, n_sink, rope, q.shape[-1], lse, qk_norm, keys_prepared)
    rc = _lib.gqa_attn_prefill_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  *dims, int(bool(causal)), cu_ptr, msl, ctypes.byref(opt),
                                  _dtype_code(q), _stream(stream))
    _check(rc, "gqa_attn_prefill_ex")
    return out


def gqa_attn_prefill_gva(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                         window: int = 0, n_sink: int = 0, scale: Optional[float] = None,
                         cu_seqlens: Optional[torch.Tensor] = None,
                         max_seqlen: Optional[int] = None, out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Grouped value attention: q, k [B,Tq|Tkv,H,d] shared by the HV = G*H value heads of
    v [B,Tkv,HV,d]; value head j uses query/key head j // G. Returns out [B,Tq,HV,d]. bf16."""
    q, k, v = _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected q[B,Tq,H,d], k[B,Tkv,H,d], v[B,Tkv,HV,d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    B, Tq, H, d = q.shape
    Tkv, HV = k.shape[1], v.shape[2]
    if k.shape[0] != B or k.shape[2] != H or k.shape[3] != d or v.shape[:2] != k.shape[:2] \
            or v.shape[3] != d:
        raise ValueError("q, k and v disagree on batch, length, heads or head dim")
    if scale is None:
        scale = GQA_SCALE_DEFAULT
    cu_ptr, nseq, msl = None, B, 0
    if cu_seqlens is not None:
        cu = _dev(cu_seqlens, "cu_seqlens")
        if cu.dtype != torch.int32 or cu.dim() != 1 or cu.numel() < 2 or B != 1:
            raise ValueError("packed batches: int32 cu_seqlens and [1, total, ., d] tensors")
        nseq = cu.numel() - 1
        cu_ptr, msl = cu.data_ptr(), _max_seqlen(max_seqlen)
    oshape = (B, Tq, HV, d)
    if out is None:
        out = torch.empty(oshape, dtype=q.dtype, device=q.device)
    elif tuple(out.shape) != oshape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor [B, Tq, HV, d] of q's dtype")
    if lse is not None:
        lse = _dev(lse, "lse")
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Tq, H) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 device tensor [B, Tq, H]")
    opt = _options(window, n_sink, None, d, lse)
    rc = _lib.gqa_attn_prefill_gva(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   nseq, Tq, Tkv, H, HV, d, float(scale), int(bool(causal)),
                                   cu_ptr, msl, ctypes.byref(opt), _dtype_code(q), _stream(stream))
    _check(rc, "gqa_attn_prefill_gva")
    return out


def gqa_prepare_keys(k: torch.Tensor, rope=None, qk_norm=None, pos0: int = 0,
                     cu_seqlens: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None,
                     out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """QK-norm (qk_norm = (w_q or None, w_k, eps); only w_k is used) then the rotary turn of
    every key row of k [B, T, Hkv, d] (packed: [1, total, Hkv, d] with cu_seqlens); key j of a
    sequence at position pos0 + j. out may be k itself. bf16."""
    k = _dev(k, "k")
    if k.dim() != 4:
        raise ValueError("expected k[B, T, Hkv, d]")
    B, T, H, d = k.shape
    nseq, cu_ptr, msl = B, None, 0
    if cu_seqlens is not None:
        cu = _dev(cu_seqlens, "cu_seqlens")
        if cu.dtype != torch.int32 or cu.dim() != 1 or cu.numel() < 2 or B != 1:
            raise ValueError("packed keys: int32 cu_seqlens and k of shape [1, total, Hkv, d]")
        nseq = cu.numel() - 1
        cu_ptr, msl = cu.data_ptr(), _max_seqlen(max_seqlen)
    if out is None:
        out = torch.empty_like(k)
    elif out.shape != k.shape or out.dtype != k.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like k")
    opt = _options(0, 0, rope, d, None, qk_norm)
    rc = _lib.gqa_prepare_keys(k.data_ptr(), out.data_ptr(), nseq, T, H, d, cu_ptr, msl,
                               int(pos0), ctypes.byref(opt), _dtype_code(k), _stream(stream))
    _check(rc, "gqa_prepare_keys")
    return out


def gqa_attn_decode_workspace_bytes(B: int, Tkv: int, Hq: int, d: int) -> int:
    """Workspace bytes enough for a decode of these sizes with any Hkv that divides Hq."""
    return int(_lib.gqa_attn_decode_workspace_bytes(B, Tkv, Hq, d))


def gqa_attn_decode_workspace_bytes_hkv(B: int, Tkv: int, Hq: int, Hkv: int, d: int) -> int:
    """The exact workspace bytes a decode with Hkv key/value heads needs."""
    return int(_lib.gqa_attn_decode_workspace_bytes_hkv(B, Tkv, Hq, Hkv, d))


def _decode_args(q, k_cache, v_cache, scale, workspace, out, workspace_needed=True):
    q, k, v = _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache")
    if q.dim() != 4 or q.shape[1] != 1 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q[B,1,Hq,d] and k_cache, v_cache[B,Tkv,Hkv,d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q and the caches must share a dtype")
    B, _, Hq, d = q.shape
    Bk, Tkv, Hkv, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError("q and the caches disagree on batch or head dim")
    if scale is None:
        scale = GQA_SCALE_DEFAULT
    ws_ptr, ws_bytes = None, 0
    if q.dtype == torch.bfloat16 and workspace_needed:
        need = gqa_attn_decode_workspace_bytes_hkv(B, Tkv, Hq, Hkv, d)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        elif workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous device tensor shaped and typed like q")
    return q, k, v, out, (B, Tkv, Hq, Hkv, d, float(scale)), ws_ptr, ws_bytes, workspace


def gqa_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    scale: Optional[float] = None, causal: bool = False,
                    workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """q [B,1,Hq,d], caches [B,Tkv,Hkv,d]; workspace: a device tensor of at least
    gqa_attn_decode_workspace_bytes(...) bytes (allocated here when None)."""
    q, k, v, out, dims, ws_ptr, ws_bytes, _ = _decode_args(q, k_cache, v_cache, scale, workspace,
                                                           out)
    rc = _lib.gqa_attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), *dims,
                              int(bool(causal)), ws_ptr, ws_bytes, _dtype_code(q),
                              _stream(stream))
    _check(rc, "gqa_attn_decode")
    return out


def gqa_attn_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            scale: Optional[float] = None, causal: bool = False,
                            out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """:func:`gqa_attn_decode` with the split partials in the library's fixed per-GPU scratch
    (no workspace; the call allocates nothing when ``out`` is given). Calls that overlap on one
    GPU share that scratch and race."""
    q, k, v, out, dims, _, _, _ = _decode_args(q, k_cache, v_cache, scale, None, out,
                                               workspace_needed=False)
    rc = _lib.gqa_attn_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      *dims, int(bool(causal)), _dtype_code(q), _stream(stream))
    _check(rc, "gqa_attn_decode_noalloc")
    return out


def gqa_attn_decode_ragged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           cache_lens: Optional[torch.Tensor] = None, window: int = 0,
                           n_sink: int = 0, scale: Optional[float] = None,
                           workspace: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode where sequence b uses cache entries 0 .. cache_lens[b]-1 (int32 device tensor;
    None: all), optionally limited to its last `window` entries plus the first n_sink; bf16."""
    q, k, v, out, dims, ws_ptr, ws_bytes, _ = _decode_args(q, k_cache, v_cache, scale, workspace,
                                                           out)
    lens_ptr = None
    if cache_lens is not None:
        lens = _dev(cache_lens, "cache_lens")
        if lens.dtype != torch.int32 or lens.dim() != 1 or lens.numel() != q.shape[0]:
            raise ValueError("cache_lens must be a 1-D int32 device tensor with one entry per "
                             "sequence")
        lens_ptr = lens.data_ptr()
    rc = _lib.gqa_attn_decode_ragged(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     *dims, lens_ptr, int(window), int(n_sink), ws_ptr, ws_bytes,
                                     _dtype_code(q), _stream(stream))
    _check(rc, "gqa_attn_decode_ragged")
    return out


def gqa_attn_decode_ex(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       cache_lens: Optional[torch.Tensor] = None, window: int = 0,
                       n_sink: int = 0, rope=None, scale: Optional[float] = None,
                       workspace: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None, qk_norm=None,
                       stream=None) -> torch.Tensor:
    """:func:`gqa_attn_decode_ragged` plus rotary embedding and QK-norm of the query (the cache
    holds processed keys); rope = (cos, sin) float32 device tables [rows >= Tmax, d/2];
    qk_norm = (w_q, w_k, eps). bf16 only."""
    q, k, v, out, dims, ws_ptr, ws_bytes, _ = _decode_args(q, k_cache, v_cache, scale, workspace,
                                                           out)
    lens_ptr = None
    if cache_lens is not None:
        lens = _dev(cache_lens, "cache_lens")
        if lens.dtype != torch.int32 or lens.dim() != 1 or lens.numel() != q.shape[0]:
            raise ValueError("cache_lens must be a 1-D int32 device tensor with one entry per "
                             "sequence")
        lens_ptr = lens.data_ptr()
    opt = _options(window, n_sink, rope, q.shape[-1], None, qk_norm)
    rc = _lib.gqa_attn_decode_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), *dims,
                                 lens_ptr, ctypes.byref(opt), ws_ptr, ws_bytes, _dtype_code(q),
                                 _stream(stream))
    _check(rc, "gqa_attn_decode_ex")
    return out


def gqa_attn_decode_window_cache(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                 cache_lens: torch.Tensor, window: int, n_sink: int = 0,
                                 rope=None, scale: Optional[float] = None,
                                 workspace: Optional[torch.Tensor] = None,
                                 out: Optional[torch.Tensor] = None, qk_norm=None,
                                 stream=None) -> torch.Tensor:
    """Decode against caches bounded to the window: k_cache, v_cache [B, n_sink + window, Hkv, d]
    with entry e of a sequence in slot e (e < n_sink) or n_sink + (e - n_sink) % window;
    cache_lens (int32 device [B]) counts every entry a sequence has had. rope / qk_norm as for
    :func:`gqa_attn_decode_ex`. bf16 only."""
    if window < 1 or n_sink < 0:
        raise ValueError("window must be >= 1 and n_sink >= 0")
    if k_cache.dim() != 4 or k_cache.shape[1] != n_sink + window:
        raise ValueError("k_cache, v_cache must hold n_sink + window slots per sequence")
    q, k, v, out, dims, ws_ptr, ws_bytes, _ = _decode_args(q, k_cache, v_cache, scale, workspace,
                                                           out)
    lens = _dev(cache_lens, "cache_lens")
    if lens.dtype != torch.int32 or lens.dim() != 1 or lens.numel() != q.shape[0]:
        raise ValueError("cache_lens must be a 1-D int32 device tensor with one entry per "
                         "sequence")
    B, _, Hq, Hkv, d, sc = dims
    opt = _options(window, n_sink, rope, d, None, qk_norm)
    rc = _lib.gqa_attn_decode_window_cache(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           out.data_ptr(), B, Hq, Hkv, d, sc, lens.data_ptr(),
                                           ctypes.byref(opt), ws_ptr, ws_bytes, _dtype_code(q),
                                           _stream(stream))
    _check(rc, "gqa_attn_decode_window_cache")
    return out


def gqa_attn_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                      dout: torch.Tensor, lse: torch.Tensor, causal: bool = False,
                      scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                      window: int = 0, n_sink: int = 0, cu_seqlens: Optional[torch.Tensor] = None,
                      max_seqlen: Optional[int] = None, stream=None):
    """Gradients (dq, dk, dv) of sum(out * dout) for a forward with the same arguments; lse from
    :func:`gqa_attn_prefill_ex`. bf16. A sliding window / sinks (causal) and packed batches
    ([1, total, H, d] with int32 device cu_seqlens and the host max_seqlen) as in the forward."""
    q, k, v = _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    out, dout, lse = _dev(out, "out"), _dev(dout, "dout"), _dev(lse, "lse")
    if q.dim() != 4 or k.shape != v.shape or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("expected q, out, dout [B,Tq,Hq,d] and k, v [B,Tkv,Hkv,d]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must be float32 [B, Tq, Hq]")
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise TypeError("q, k, v, out and dout must share a dtype")
    B, Tq, Hq, d = q.shape
    if k.dim() != 4 or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must be [B, Tkv, Hkv, d] with q's batch and head dim")
    Tkv, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = GQA_SCALE_DEFAULT
    nseq, cu_ptr, msl = B, None, 0
    if cu_seqlens is not None:
        cu = _dev(cu_seqlens, "cu_seqlens")
        if cu.dtype != torch.int32 or cu.dim() != 1 or cu.numel() < 2 or B != 1:
            raise ValueError("packed batches: int32 cu_seqlens and [1, total, H, d] tensors")
        nseq = cu.numel() - 1
        cu_ptr, msl = cu.data_ptr(), _max_seqlen(max_seqlen)
    need = int(_lib.gqa_attn_backward_workspace_bytes(B, Tq, Hq))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), nseq, Tq, Tkv, Hq, Hkv,
            d, float(scale), int(bool(causal)))
    ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    if window or n_sink or cu_seqlens is not None:
        opt = _options(window, n_sink, None, d)
        rc = _lib.gqa_attn_backward_ex(*args, cu_ptr, msl, ctypes.byref(opt), *ws, _dtype_code(q),
                                       _stream(stream))
        _check(rc, "gqa_attn_backward_ex")
    else:
        rc = _lib.gqa_attn_backward(*args, *ws, _dtype_code(q), _stream(stream))
        _check(rc, "gqa_attn_backward")
    return dq, dk, dv


def gqa_fold_kv(src: torch.Tensor, g: int, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """src [B,T,H,d] -> [B,T,g,d], mean over contiguous groups of H/g heads."""
    if not isinstance(src, torch.Tensor) or src.dim() != 4:
        raise ValueError("expected src[B,T,H,d]")
    B, T, H, d = src.shape
    if g <= 0 or H % g != 0:
        raise GQAValueError(GQA_ERR_GROUPING, f"{H} heads do not fold evenly into {g} groups")
    src = _dev(src, "src")
    if out is None:
        out = torch.empty((B, T, g, d), dtype=src.dtype, device=src.device)
    elif tuple(out.shape) != (B, T, g, d) or out.dtype != src.dtype or not out.is_contiguous() \
            or out.device != src.device:
        raise ValueError("out must be a contiguous device tensor [B, T, g, d] of src's dtype")
    rc = _lib.gqa_fold_kv(src.data_ptr(), out.data_ptr(), B, T, H, g, d, _dtype_code(src),
                          _stream(stream))
    _check(rc, "gqa_fold_kv")
    return out


def raw_library() -> ctypes.CDLL:
    return _lib
