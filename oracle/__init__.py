"""fp64 CPU oracle for grouped-query attention forward (Python face of ``gqa_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the benchmark's
CPU-baseline leg. The HIP library and its Python binding never import it.

Functions mirror the GQA lab page ("Transformer -- attention by hand: reducing only the key/value
heads"): ``group_of`` / ``group_members`` (step 1), ``fold_kv`` (step 2), ``expand_kv`` (step 3),
``attention`` (step 4 per head, run over all heads as in step 5's ``heads_out``), ``max_gap``
(step 5), and the counts ``kv_cache_elems`` / ``kv_table`` / ``mults`` (steps 6-7, in
:mod:`oracle.counts`). As on the page, a head count that does not divide evenly raises
``ValueError``. ``window_cache_slot`` / ``window_cache_visible`` / ``unroll_window_cache`` read a
decode cache bounded to the sliding window (course page "Week 7. Attention", step 3) back in
arrival order, for ``attention`` to run on.

Array conventions: numpy arrays; float64 and float32 are taken as values, uint16 as bfloat16 bit
patterns. Outputs are float64.

Parity pins (tests/test_oracle_pins.py) tie every function to the pages' worked examples, closed
forms, invariants and torch's CPU fp64 ``scaled_dot_product_attention``; see that file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

from .counts import kv_cache_elems, kv_table, mults  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_F64, _F32, _BF16 = 0, 1, 2
_ERRORS = {1: ValueError, 2: ValueError, 3: MemoryError}
_ERRMSG = {1: "head count is not divisible by the group count",
           2: "invalid shape or index", 3: "out of memory"}


def build(out_path: str = _LIB_PATH, extra_flags: Sequence[str] = ()) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP). Returns the shared-object path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", *extra_flags, _SRC,
           "-o", out_path + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


_lib = None


def _load(path: Optional[str] = None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib):
    P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_group_of.argtypes = [I, I, I]
    lib.oracle_group_of.restype = I
    lib.oracle_fold.argtypes = [P, I, P, I64, I64, I, I, I]
    lib.oracle_fold.restype = I
    lib.oracle_expand.argtypes = [P, P, I64, I64, I, I, I]
    lib.oracle_expand.restype = I
    lib.oracle_gqa_attention.argtypes = [P, P, P, I, P, I64, I64, I64, I, I, I, D, I, P, I, I64,
                                         I64, P, P, I64, I, P, P, D]
    lib.oracle_gqa_attention.restype = I
    lib.oracle_gqa_attention_rows.argtypes = [P, P, P, I, I64, I64, I64, I, I, I, D, I, P, I, P,
                                              I64, P, I64, I64, P, P, I64, I, P, P, D]
    lib.oracle_gqa_attention_rows.restype = I
    lib.oracle_gqa_attention_bwd.argtypes = [P, P, P, P, I, P, P, P, I64, I64, I64, I, I, I, D,
                                             I, I64, I64]
    lib.oracle_gqa_attention_bwd.restype = I
    lib.oracle_gva_attention.argtypes = [P, P, P, I, P, I64, I64, I64, I, I, I, D, I, P, I, I64,
                                         I64]
    lib.oracle_gva_attention.restype = I
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = I
    return lib


class Oracle:
    """Bound oracle; :data:`default` uses the in-tree build. Tests may bind another build."""

    def __init__(self, lib_path: Optional[str] = None):
        self.lib = _load(lib_path)

    # -- helpers ----------------------------------------------------------------------------
    @staticmethod
    def _prep(a: np.ndarray):
        a = np.ascontiguousarray(a)
        if a.dtype == np.float64:
            return a, _F64
        if a.dtype == np.float32:
            return a, _F32
        if a.dtype == np.uint16:
            return a, _BF16
        raise TypeError(f"unsupported oracle input dtype {a.dtype}")

    @staticmethod
    def _check(rc: int):
        if rc:
            raise _ERRORS.get(rc, RuntimeError)(_ERRMSG.get(rc, f"oracle error {rc}"))

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    # -- lab step 1 -------------------------------------------------------------------------
    def group_of(self, head: int, h: int, g: int) -> int:
        if g <= 0 or h <= 0 or h % g != 0:
            raise ValueError(f"{h} heads do not split evenly into {g} groups")
        r = self.lib.oracle_group_of(head, h, g)
        if r < 0:
            raise ValueError(f"head {head} out of range for {h} heads")
        return r

    def group_members(self, h: int, g: int) -> List[List[int]]:
        """Members of each group, filled by calling :meth:`group_of` once per head."""
        if g <= 0 or h <= 0 or h % g != 0:
            raise ValueError(f"{h} heads do not split evenly into {g} groups")
        groups: List[List[int]] = [[] for _ in range(g)]
        for head in range(h):
            groups[self.group_of(head, h, g)].append(head)
        return groups

    # -- lab steps 2, 3 ---------------------------------------------------------------------
    def fold_kv(self, x: np.ndarray, g: int) -> np.ndarray:
        """x[B,T,H,d] -> float64 [B,T,g,d], mean over each contiguous group of H/g heads."""
        x, dt = self._prep(x)
        B, T, H, d = x.shape
        out = np.empty((B, T, g, d), dtype=np.float64) if g > 0 else None
        if g <= 0 or H % g != 0:
            raise ValueError(f"{H} heads do not fold evenly into {g} groups")
        self._check(self.lib.oracle_fold(x.ctypes.data, dt, out.ctypes.data, B, T, H, g, d))
        return out

    def expand_kv(self, folded: np.ndarray, h: int) -> np.ndarray:
        """folded[B,T,g,d] -> float64 [B,T,h,d] by adjacent repetition ([A,B] -> [A,A,B,B])."""
        f = np.ascontiguousarray(folded, dtype=np.float64)
        B, T, g, d = f.shape
        if h <= 0 or h % g != 0:
            raise ValueError(f"{g} heads do not expand evenly to {h}")
        out = np.empty((B, T, h, d), dtype=np.float64)
        self._check(self.lib.oracle_expand(f.ctypes.data, out.ctypes.data, B, T, g, h, d))
        return out

    # -- lab steps 4, 5 ---------------------------------------------------------------------
    def _common(self, q, k, v, scale, cu_seqlens):
        q, dq = self._prep(q)
        k, dk = self._prep(k)
        v, dv = self._prep(v)
        if not (dq == dk == dv):
            raise TypeError("q, k and v must share a dtype")
        if q.ndim != 4 or k.ndim != 4 or v.ndim != 4 or k.shape != v.shape:
            raise ValueError("expected q[B,Tq,Hq,d], k,v[B,Tkv,Hkv,d]")
        B, Tq, Hq, d = q.shape
        Bk, Tkv, Hkv, dk_ = k.shape
        if Bk != B or dk_ != d:
            raise ValueError("q and k/v disagree on batch or head dim")
        if Hkv <= 0 or Hq % Hkv != 0:
            raise ValueError(f"{Hq} query heads do not group evenly over {Hkv} key/value heads")
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        cu = None
        nseq = 0
        if cu_seqlens is not None:
            cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
            nseq = len(cu) - 1
            if B != 1 or Tq != Tkv or cu[-1] != Tq:
                raise ValueError("packed batch needs q,k,v as [1,total,H,d] with total == cu[-1]")
        return q, k, v, dq, B, Tq, Tkv, Hq, Hkv, d, float(scale), cu, nseq

    @staticmethod
    def _rope(rope, rope_mode, d):
        """rope: None or (cos, sin) float32 tables [n_pos, d/2]; rope_mode "qk" rotates queries
        and keys, "q" only the queries (keys already rotated, as in a cache)."""
        if rope is None:
            return None, None, 0, 0, ()
        cos_t = np.ascontiguousarray(rope[0], dtype=np.float32)
        sin_t = np.ascontiguousarray(rope[1], dtype=np.float32)
        if cos_t.shape != sin_t.shape or cos_t.ndim != 2 or cos_t.shape[1] * 2 != d:
            raise ValueError("rope tables must both be [n_pos, d/2]")
        mode = {"qk": 3, "q": 1}[rope_mode]
        return cos_t.ctypes.data, sin_t.ctypes.data, cos_t.shape[0], mode, (cos_t, sin_t)

    @staticmethod
    def _norm(qk_norm, qk_norm_mode, d):
        """qk_norm: None or (w_q, w_k, eps) with float32 weights [d]; qk_norm_mode "qk" normalises
        queries and keys, "q" only the queries (keys already normalised, as in a cache)."""
        if qk_norm is None:
            return None, None, 0.0, ()
        wq = np.ascontiguousarray(qk_norm[0], dtype=np.float32)
        wk = np.ascontiguousarray(qk_norm[1], dtype=np.float32)
        if wq.shape != (d,) or wk.shape != (d,):
            raise ValueError("qk-norm weights must be float32 [d]")
        kp = wk.ctypes.data if qk_norm_mode == "qk" else None
        return wq.ctypes.data, kp, float(qk_norm[2]), (wq, wk)

    def attention(self, q, k, v, scale: Optional[float] = None, causal: bool = False,
                  cu_seqlens=None, window: int = 0, n_sink: int = 0, rope=None,
                  rope_mode: str = "qk", qk_norm=None, qk_norm_mode: str = "qk") -> np.ndarray:
        """Grouped-query attention forward (``heads_out``): float64 out[B,Tq,Hq,d].

        ``window`` > 0 (causal only) limits each query at position p to keys p-window+1 .. p,
        plus the ``n_sink`` first keys; ``rope`` = (cos, sin) tables rotates query t at position
        t + Tkv - Tq and key j at position j before the scores (course page "Week 7. Attention",
        step 3). ``qk_norm`` = (w_q, w_k, eps) applies RMSNorm with those weights to every query
        and key head row before the rotation (course page, step 3: QK-norm)."""
        q, k, v, dt, B, Tq, Tkv, Hq, Hkv, d, scale, cu, nseq = self._common(q, k, v, scale,
                                                                            cu_seqlens)
        cp, sp, npos, mode, keep = self._rope(rope, rope_mode, d)
        qn, kn, eps, keep2 = self._norm(qk_norm, qk_norm_mode, d)
        out = np.empty((B, Tq, Hq, d), dtype=np.float64)
        rc = self.lib.oracle_gqa_attention(q.ctypes.data, k.ctypes.data, v.ctypes.data, dt,
                                           out.ctypes.data, B, Tq, Tkv, Hq, Hkv, d, scale,
                                           int(bool(causal)),
                                           cu.ctypes.data if cu is not None else None, nseq,
                                           int(window), int(n_sink), cp, sp, npos, mode, qn, kn,
                                           eps)
        del keep, keep2
        self._check(rc)
        return out

    def attention_rows(self, q, k, v, rows: np.ndarray, scale: Optional[float] = None,
                       causal: bool = False, cu_seqlens=None, window: int = 0,
                       n_sink: int = 0, rope=None, rope_mode: str = "qk", qk_norm=None,
                       qk_norm_mode: str = "qk") -> np.ndarray:
        """Selected output rows only. rows: int64 [n, 3] of (b, t, head); returns float64 [n, d]."""
        q, k, v, dt, B, Tq, Tkv, Hq, Hkv, d, scale, cu, nseq = self._common(q, k, v, scale,
                                                                            cu_seqlens)
        r = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
        cp, sp, npos, mode, keep = self._rope(rope, rope_mode, d)
        qn, kn, eps, keep2 = self._norm(qk_norm, qk_norm_mode, d)
        out = np.empty((r.shape[0], d), dtype=np.float64)
        rc = self.lib.oracle_gqa_attention_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data, dt,
                                                B, Tq, Tkv, Hq, Hkv, d, scale, int(bool(causal)),
                                                cu.ctypes.data if cu is not None else None, nseq,
                                                r.ctypes.data, r.shape[0], out.ctypes.data,
                                                int(window), int(n_sink), cp, sp, npos, mode, qn,
                                                kn, eps)
        del keep, keep2
        self._check(rc)
        return out

    def attention_bwd(self, q, k, v, dout, scale: Optional[float] = None, causal: bool = False,
                      window: int = 0, n_sink: int = 0):
        """Gradients (dq, dk, dv) of sum(out * dout) for the forward :meth:`attention`, float64.
        dk / dv sum the contributions of the G query heads that share each key/value head."""
        q, k, v, dt, B, Tq, Tkv, Hq, Hkv, d, scale, _, _ = self._common(q, k, v, scale, None)
        g, dtg = self._prep(dout)
        if dtg != dt or g.shape != q.shape:
            raise ValueError("dout must match q in shape and dtype")
        dq = np.empty((B, Tq, Hq, d), dtype=np.float64)
        dk = np.empty((B, Tkv, Hkv, d), dtype=np.float64)
        dv = np.empty((B, Tkv, Hkv, d), dtype=np.float64)
        rc = self.lib.oracle_gqa_attention_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                               g.ctypes.data, dt, dq.ctypes.data, dk.ctypes.data,
                                               dv.ctypes.data, B, Tq, Tkv, Hq, Hkv, d, scale,
                                               int(bool(causal)), int(window), int(n_sink))
        self._check(rc)
        return dq, dk, dv

    def attention_gva(self, q, k, v, scale: Optional[float] = None, causal: bool = False,
                      cu_seqlens=None, window: int = 0, n_sink: int = 0) -> np.ndarray:
        """Grouped value attention (K3 notes, section 4): q, k [B,T,H,d] shared by the
        HV = G*H value heads of v [B,Tkv,HV,d]; value head j uses query/key head j // G.
        Returns float64 out[B,Tq,HV,d]."""
        q, dq = self._prep(q)
        k, dk = self._prep(k)
        v, dv = self._prep(v)
        if not (dq == dk == dv):
            raise TypeError("q, k and v must share a dtype")
        if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
            raise ValueError("expected q[B,Tq,H,d], k[B,Tkv,H,d], v[B,Tkv,HV,d]")
        B, Tq, H, d = q.shape
        if k.shape[0] != B or k.shape[2] != H or k.shape[3] != d or v.shape[:2] != k.shape[:2] \
                or v.shape[3] != d:
            raise ValueError("q, k and v disagree on batch, length, heads or head dim")
        Tkv, HV = k.shape[1], v.shape[2]
        if HV % H != 0:
            raise ValueError(f"{HV} value heads do not group evenly over {H} query/key heads")
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        cu, nseq = None, 0
        if cu_seqlens is not None:
            cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
            nseq = len(cu) - 1
            if B != 1 or Tq != Tkv or cu[-1] != Tq:
                raise ValueError("packed batch needs [1,total,H,d] inputs with total == cu[-1]")
        out = np.empty((B, Tq, HV, d), dtype=np.float64)
        rc = self.lib.oracle_gva_attention(q.ctypes.data, k.ctypes.data, v.ctypes.data, dq,
                                           out.ctypes.data, B, Tq, Tkv, H, HV, d, float(scale),
                                           int(bool(causal)),
                                           cu.ctypes.data if cu is not None else None, nseq,
                                           int(window), int(n_sink))
        self._check(rc)
        return out

    def heads_out(self, q, k, v, g: int, causal: bool = False) -> np.ndarray:
        """The lab's three-way protocol: fold K and V to g heads, then attend with all query heads."""
        kf = self.fold_kv(k, g)
        vf = self.fold_kv(v, g)
        return self.attention(np.asarray(q, dtype=np.float64) if q.dtype != np.uint16 else
                              _bf16_to_f64(q), kf, vf, causal=causal)


def _window_slots(entries: np.ndarray, window: int, n_sink: int) -> np.ndarray:
    """Slots of cache entries in a cache bounded to the window: an entry below n_sink keeps its
    own slot; a later entry e goes to slot n_sink + (e - n_sink) mod window, the slot of the entry
    `window` places before it, which has left the window (course page "Week 7. Attention",
    step 3: the window bounds the cache to its size, and the sink tokens are never dropped)."""
    e = np.asarray(entries, dtype=np.int64)
    return np.where(e < n_sink, e, n_sink + (e - n_sink) % window)


def window_cache_slot(entry: int, window: int, n_sink: int) -> int:
    """Slot (0 .. n_sink + window - 1) that keeps cache entry ``entry`` (0-based, in arrival
    order) of a cache bounded to ``window`` entries plus ``n_sink`` sink entries."""
    if window < 1 or n_sink < 0 or entry < 0:
        raise ValueError("window_cache_slot: window >= 1, n_sink >= 0, entry >= 0")
    return int(_window_slots(np.array([entry]), window, n_sink)[0])


def window_cache_visible(length: int, window: int, n_sink: int) -> np.ndarray:
    """Entries that the newest query of a sequence of ``length`` entries sees (it sits at
    position length - 1): the sinks 0 .. n_sink - 1 and the last ``window`` entries (course
    page, step 3; the same visibility as ``attention(..., causal=True, window, n_sink)``)."""
    e = np.arange(max(int(length), 0), dtype=np.int64)
    return e[(e < n_sink) | (e >= length - window)]


def unroll_window_cache(ring: np.ndarray, lengths, window: int, n_sink: int,
                        compact: bool = False) -> List[np.ndarray]:
    """Each sequence's cache in arrival order, read out of its window-bounded cache
    ``ring`` [B, n_sink + window, Hkv, d]: every visible entry from its slot.

    compact=False: [1, length, Hkv, d] with the entries that the window hides set to zero (they
    are never looked at by a windowed query at position length - 1); compact=True: only the
    visible entries, in arrival order, [1, n_visible, Hkv, d]."""
    ring = np.asarray(ring)
    if window < 1 or n_sink < 0 or ring.ndim != 4 or ring.shape[1] != n_sink + window:
        raise ValueError("unroll_window_cache: ring must be [B, n_sink + window, Hkv, d]")
    if len(lengths) != ring.shape[0]:
        raise ValueError("unroll_window_cache: one length per sequence")
    out = []
    for b, length in enumerate(lengths):
        vis = window_cache_visible(length, window, n_sink)
        rows = ring[b, _window_slots(vis, window, n_sink)]
        if compact:
            out.append(rows[None].copy())
        else:
            full = np.zeros((1, max(int(length), 0)) + ring.shape[2:], dtype=ring.dtype)
            full[0, vis] = rows
            out.append(full)
    return out


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def max_gap(left: np.ndarray, right: np.ndarray) -> float:
    """Largest absolute elementwise difference over every head, row and column (lab step 5)."""
    a = np.asarray(left, dtype=np.float64)
    b = np.asarray(right, dtype=np.float64)
    if a.shape != b.shape:
        raise ValueError("max_gap: shapes differ")
    return float(np.max(np.abs(a - b))) if a.size else 0.0


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
