"""Exact integer counts from the GQA lab page (steps 6 and 7). TEST INFRASTRUCTURE ONLY.

* KV cache size, counted in elements (not bytes, because an element is 2 or 4 bytes depending on
  the dtype): two tensors (K and V) x layers x key/value heads x length x head dim. The number of
  query heads does not appear, because queries are not cached.
* Multiplies for one pass of one layer, per term: each projection costs
  tokens x model width x (its head count x head dim); the score and weighted-sum terms each cost
  query heads x tokens x tokens x head dim. Only the K and V projections depend on the group
  count g. Additions and softmax exponentials are not counted.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Tuple


def _check_groups(h: int, g: int) -> None:
    if g <= 0 or h <= 0 or h % g != 0:
        raise ValueError(f"{h} heads do not split evenly into {g} groups")


def kv_cache_elems(layers: int, kv_heads: int, seq_len: int, head_dim: int) -> int:
    return 2 * layers * kv_heads * seq_len * head_dim


def kv_table(layers: int, h: int, groups: Iterable[int], seq_len: int,
             head_dim: int) -> List[Tuple[int, int]]:
    """[(g, elements)] for each group count g; with g groups there are exactly g K/V heads."""
    out = []
    for g in groups:
        _check_groups(h, g)
        out.append((g, kv_cache_elems(layers, g, seq_len, head_dim)))
    return out


def mults(n: int, d_model: int, h: int, g: int, head_dim: int) -> Dict[str, int]:
    _check_groups(h, g)
    terms = {
        "proj_q": n * d_model * (h * head_dim),
        "proj_k": n * d_model * (g * head_dim),
        "proj_v": n * d_model * (g * head_dim),
        "scores": h * n * n * head_dim,
        "weighted": h * n * n * head_dim,
        "proj_out": n * d_model * (h * head_dim),
    }
    terms["total"] = sum(terms.values())
    return terms


def core_mults(n: int, d_model: int, h: int, g: int, head_dim: int) -> int:
    """scores + weighted: the attention-core multiplies (the same for every g)."""
    m = mults(n, d_model, h, g, head_dim)
    return m["scores"] + m["weighted"]
