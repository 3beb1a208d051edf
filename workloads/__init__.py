"""Seeded synthetic inputs for grouped-query attention.

This module is shared by the CPU oracle's tests, the GPU parity tests and the benchmark. It only
draws numbers and describes shapes; it holds none of the attention arithmetic (no grouping, no
folding, no softmax), so the oracle and the HIP path stay independent of each other.

Sources for the shapes and value distributions:
  * the GQA lab page ("Transformer — attention by hand: reducing only the key/value heads",
    step 1 and its note "split the query heads into groups"): a small linear congruential
    generator that emits ``state / m - 0.5`` and fills heads head-major; seeds 101 / 202 / 303
    for q / k / v in the lab's report step (step 8);
  * the course page ("Week 7. Attention", step 2): the Llama-3-8B head configuration with
    32 query heads and 8 key/value heads, head dimension 128.
The pages do not give the generator's constants; the Numerical Recipes constants are used.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# Numerical Recipes LCG constants (the lab fixes only the form of the recurrence).
LCG_A = 1664525
LCG_C = 1013904223
LCG_M = 1 << 32


def make_heads(count: int, rows: int, dim: int, seed: int) -> np.ndarray:
    """Deterministic head tensor ``[count][rows][dim]`` in [-0.5, 0.5) as float64.

    Each draw first advances ``state = (a*state + c) % m`` and then emits ``state/m - 0.5``;
    values are filled head-major, as the lab's ``make_heads(count, rows, dim, seed)`` implies.
    """
    if count <= 0 or rows <= 0 or dim <= 0:
        raise ValueError("make_heads: sizes must be positive")
    n = count * rows * dim
    out = np.empty(n, dtype=np.float64)
    state = seed % LCG_M
    for i in range(n):
        state = (LCG_A * state + LCG_C) % LCG_M
        out[i] = state / LCG_M - 0.5
    return out.reshape(count, rows, dim)


def heads_to_bthd(heads: np.ndarray) -> np.ndarray:
    """``[H][T][d]`` head-major table -> ``[1, T, H, d]`` activation layout (a pure transpose)."""
    return np.ascontiguousarray(np.transpose(heads, (1, 0, 2))[None, ...])


# ----------------------------------------------------------------------------------------------
# bf16 helpers (bit-level; torch is used only as a seeded normal generator and for RNE rounding)
# ----------------------------------------------------------------------------------------------

def randn_f32(shape: Sequence[int], seed: int):
    """Seeded N(0,1) draws in float32 from torch's CPU generator (a torch tensor)."""
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def to_bf16(t):
    """Round-to-nearest-even float32 -> bfloat16 (torch CPU)."""
    import torch
    return t.to(torch.bfloat16)


def randn_bf16(shape: Sequence[int], seed: int):
    return to_bf16(randn_f32(shape, seed))


def bf16_bits(t) -> np.ndarray:
    """The raw 16-bit patterns of a CPU bfloat16 tensor as a numpy uint16 array (no copy of values)."""
    import torch
    assert t.dtype == torch.bfloat16 and t.device.type == "cpu"
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------------------------
# Workload descriptions
# ----------------------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Tq: int
    Tkv: int
    Hq: int
    Hkv: int
    d: int
    dtype: str            # "f32" or "bf16"
    causal: bool
    seqlens: Optional[Tuple[int, ...]] = None   # packed variable-length batch (B == 1)
    seeds: Tuple[int, int, int] = (0, 1, 2)
    peaked_frac: float = 0.0                    # fraction of q rows multiplied by peaked_scale
    peaked_scale: float = 1.0
    peaked_seed: int = 0
    window: int = 0                             # causal sliding window (0: none)
    n_sink: int = 0                             # sink keys kept visible below the window
    cache_lens: Optional[Tuple[int, ...]] = None  # ragged decode: entries used per sequence
    window_cache: bool = False  # decode cache bounded to the window: Tkv = n_sink + window slots,
                                # cache_lens count every entry a sequence has had

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def cu_seqlens(self) -> Optional[np.ndarray]:
        if self.seqlens is None:
            return None
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    @property
    def is_decode(self) -> bool:
        return self.Tq == 1 and self.Tkv > 1 and self.seqlens is None


# Tiny fp32 lab-style case: B=1, Hq=8, T=64, d=16, LCG seeds 101/202/303.
TINY = Workload("tiny_f32_lab", B=1, Tq=64, Tkv=64, Hq=8, Hkv=8, d=16, dtype="f32", causal=False,
                seeds=(101, 202, 303))
# Llama-3-8B-shaped causal prefill: 32 query / 8 kv heads, d=128, T=4096.
LLAMA_PREFILL = Workload("llama3_8b_causal_prefill_T4096", B=1, Tq=4096, Tkv=4096, Hq=32, Hkv=8,
                         d=128, dtype="bf16", causal=True, seeds=(2000, 2001, 2002))
# Batched decode: 64 sequences, one query token, 8192-entry cache.
DECODE = Workload("decode_B64_kv8192", B=64, Tq=1, Tkv=8192, Hq=32, Hkv=8, d=128, dtype="bf16",
                  causal=False, seeds=(3000, 3001, 3002))
# MQA extreme causal prefill with 5% of q rows scaled x30.
MQA_PREFILL = Workload("mqa_causal_prefill_B8_T2048", B=8, Tq=2048, Tkv=2048, Hq=32, Hkv=1, d=128,
                       dtype="bf16", causal=True, seeds=(4000, 4001, 4002), peaked_frac=0.05,
                       peaked_scale=30.0, peaked_seed=4003)
# Long-context packed variable-length causal prefill.
VARLEN_PREFILL = Workload("varlen_causal_prefill_16k_8k_4k_1k", B=1, Tq=29696, Tkv=29696, Hq=64,
                          Hkv=8, d=128, dtype="bf16", causal=True,
                          seqlens=(16384, 8192, 4096, 1024), seeds=(5000, 5001, 5002))



def rope_tables(npos: int, d: int, base: float = 10000.0) -> Tuple[np.ndarray, np.ndarray]:
    """Rotary-embedding input tables as a caller would pass them: cos / sin of p * theta_i with
    theta_i = base^(-2i/d) (course page "Week 7. Attention", step 3), evaluated in float64 and
    stored as float32 arrays [npos, d/2]."""
    i = np.arange(d // 2, dtype=np.float64)
    ang = np.arange(npos, dtype=np.float64)[:, None] * (base ** (-2.0 * i / d))[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def ragged_lengths(B: int, Tmax: int, seed: int) -> Tuple[int, ...]:
    """Seeded per-sequence cache lengths, uniform on 1 .. Tmax (a serving batch at mixed
    progress), with the extremes 1 and Tmax always present."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, Tmax + 1, size=B)
    lens[0], lens[-1] = 1, Tmax
    return tuple(int(x) for x in lens)


# Llama-3-8B-shaped prefill with a causal sliding window of 1024 keys and 4 sink keys (course
# page "Week 7. Attention", step 3) over an 8192-token sequence.
WINDOW_PREFILL = Workload("window_prefill_T8192_W1024_S4", B=1, Tq=8192, Tkv=8192, Hq=32, Hkv=8,
                          d=128, dtype="bf16", causal=True, seeds=(6000, 6001, 6002),
                          window=1024, n_sink=4)
# Batched decode against a ragged cache: 64 sequences with lengths uniform on 1 .. 8192 in
# caches allocated for 8192 entries.
RAGGED_DECODE = Workload("ragged_decode_B64_max8192", B=64, Tq=1, Tkv=8192, Hq=32, Hkv=8, d=128,
                         dtype="bf16", causal=False, seeds=(7000, 7001, 7002),
                         cache_lens=ragged_lengths(64, 8192, 7003))

# Grouped value attention (K3 notes, section 4): 16 query/key heads shared by 32 value heads
# (G = 2) of 64 dims, so one query/key head's values form one 128-column row; two 4096-token
# sequences. Hq here counts the value heads (the output heads) and Hkv the query/key heads.
GVA_PREFILL = Workload("gva_prefill_B2_T4096_H16_HV32_d64", B=2, Tq=4096, Tkv=4096, Hq=32, Hkv=16,
                       d=64, dtype="bf16", causal=True, seeds=(8000, 8001, 8002))

# Long-context decode: one sequence against a 131072-entry cache (32/8 heads, d = 128). The
# cache is split across the compute units, so the partial results go through the combine step.
LONG_DECODE = Workload("decode_B1_kv131072", B=1, Tq=1, Tkv=131072, Hq=32, Hkv=8, d=128,
                       dtype="bf16", causal=False, seeds=(9000, 9001, 9002))

# Decode against caches bounded to the window (course page "Week 7. Attention", step 3): 64
# sequences of 32768 entries each, 32/8 heads, d = 128, a window of 4096 entries and 4 sinks, so
# each cache holds 4100 slots (written over about eight times).
WINDOW_CACHE_DECODE = Workload("window_cache_decode_B64_W4096_S4", B=64, Tq=1, Tkv=4100, Hq=32,
                               Hkv=8, d=128, dtype="bf16", causal=False,
                               seeds=(9500, 9501, 9502), window=4096, n_sink=4,
                               cache_lens=(32768,) * 64, window_cache=True)

WORKLOADS: Dict[str, Workload] = {w.name: w for w in
                                  (TINY, LLAMA_PREFILL, DECODE, MQA_PREFILL, VARLEN_PREFILL,
                                   WINDOW_PREFILL, RAGGED_DECODE, GVA_PREFILL, LONG_DECODE,
                                   WINDOW_CACHE_DECODE)}


def tiny_lab_inputs(x1000: bool = False) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """q, k, v for the tiny lab case as float32 ``[1,64,8,16]`` (K/V with all 8 heads).

    With ``x1000`` every value is multiplied by 1000 in float64 before rounding to float32, the
    large-score stress input of the lab's step 4 note.
    """
    w = TINY
    out = []
    for s in w.seeds:
        h = heads_to_bthd(make_heads(w.Hq, w.Tq, w.d, s))
        if x1000:
            h = h * 1000.0
        out.append(h.astype(np.float32))
    return tuple(out)


def tiny_direct_kv(hkv: int, seeds=(202, 303)) -> Tuple[np.ndarray, np.ndarray]:
    """K/V generated directly with ``hkv`` heads (no folding), float32 ``[1,64,hkv,16]``."""
    w = TINY
    return tuple(heads_to_bthd(make_heads(hkv, w.Tkv, w.d, s)).astype(np.float32) for s in seeds)


def make_inputs(w: Workload):
    """q, k, v as CPU torch tensors in the workload's dtype, plus cu_seqlens (numpy int32 or None).

    bf16 workloads: i.i.d. N(0,1) drawn in float32 with torch's CPU generator, optionally with a
    seeded fraction of q rows (a row is one vector q[b,t,h,:]) multiplied in float32, then rounded
    to bf16 (round-to-nearest-even).
    """
    import torch
    if w.dtype == "f32":
        q, k, v = (torch.from_numpy(a) for a in tiny_lab_inputs())
        return q, k, v, None
    total_q = sum(w.seqlens) if w.seqlens else w.Tq
    total_k = sum(w.seqlens) if w.seqlens else w.Tkv
    qf = randn_f32((w.B, total_q, w.Hq, w.d), w.seeds[0])
    if w.peaked_frac > 0:
        nrows = w.B * total_q * w.Hq
        nsel = int(round(w.peaked_frac * nrows))
        g = torch.Generator(device="cpu")
        g.manual_seed(w.peaked_seed)
        sel = torch.randperm(nrows, generator=g)[:nsel]
        flat = qf.view(nrows, w.d)
        flat[sel] *= w.peaked_scale
    q = to_bf16(qf)
    del qf
    k = randn_bf16((w.B, total_k, w.Hkv, w.d), w.seeds[1])
    v = randn_bf16((w.B, total_k, w.Hkv, w.d), w.seeds[2])
    return q, k, v, w.cu_seqlens


def peaked_rows(w: Workload) -> np.ndarray:
    """Flat indices (b*T*Hq + t*Hq + h) of the q rows that :func:`make_inputs` scales."""
    import torch
    if w.peaked_frac <= 0:
        return np.zeros(0, dtype=np.int64)
    nrows = w.B * w.Tq * w.Hq
    nsel = int(round(w.peaked_frac * nrows))
    g = torch.Generator(device="cpu")
    g.manual_seed(w.peaked_seed)
    return torch.randperm(nrows, generator=g)[:nsel].numpy().astype(np.int64)


def gva_inputs(w: Workload):
    """q, k [B, T, H, d] and v [B, T, HV, d] as CPU bf16 tensors for a grouped value attention
    workload (H = w.Hkv query/key heads, HV = w.Hq value heads), N(0,1) with the workload seeds."""
    H, HV = w.Hkv, w.Hq
    q = randn_bf16((w.B, w.Tq, H, w.d), w.seeds[0])
    k = randn_bf16((w.B, w.Tkv, H, w.d), w.seeds[1])
    v = randn_bf16((w.B, w.Tkv, HV, w.d), w.seeds[2])
    return q, k, v


def sample_rows(w: Workload, n: int, seed: int) -> np.ndarray:
    """A seeded sample of output rows as an int64 array ``[n', 3]`` of (b, t, head).

    Always contains the first and last query position of every batch item (or packed sequence)
    for the first and last head, so tile boundaries and the longest causal rows are covered.
    """
    rng = np.random.default_rng(seed)
    rows: List[Tuple[int, int, int]] = []
    if w.seqlens is not None:
        cu = w.cu_seqlens
        for s in range(len(w.seqlens)):
            for t in (int(cu[s]), int(cu[s + 1]) - 1):
                for h in (0, w.Hq - 1):
                    rows.append((0, t, h))
        tot = int(cu[-1])
        for _ in range(n):
            rows.append((0, int(rng.integers(tot)), int(rng.integers(w.Hq))))
    else:
        for b in sorted({0, w.B - 1}):
            for t in sorted({0, w.Tq - 1}):
                for h in (0, w.Hq - 1):
                    rows.append((b, t, h))
        for _ in range(n):
            rows.append((int(rng.integers(w.B)), int(rng.integers(w.Tq)), int(rng.integers(w.Hq))))
    arr = np.unique(np.array(rows, dtype=np.int64), axis=0)
    return arr
