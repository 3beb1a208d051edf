"""The oracle against its pins (CPU only): worked examples, closed forms, invariants and torch's
CPU fp64 scaled_dot_product_attention. The checks and their page citations live in
``oracle_pin_checks.py``."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import counts
import oracle_pin_checks as pins

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(orc, check):
    check(orc)


@pytest.mark.parametrize("check", pins.COUNT_CHECKS, ids=lambda c: c.__name__)
def test_count_pin(check):
    check(counts)


def test_fold_and_expand_reject_uneven(orc):
    x = np.zeros((1, 2, 8, 4))
    with pytest.raises(ValueError):
        orc.fold_kv(x, 3)
    with pytest.raises(ValueError):
        orc.expand_kv(np.zeros((1, 2, 3, 4)), 8)
    with pytest.raises(ValueError):
        orc.attention(np.zeros((1, 2, 8, 4)), np.zeros((1, 2, 3, 4)), np.zeros((1, 2, 3, 4)))


def test_lab_counts_against_page_ratios():
    """Lab steps 6-8 and course step 2: the cache shrinks with the K/V head count (up to 8x at
    the lab scale, 4x for 32/8 heads, 32x for MQA) while the attention-core multiplies do not
    depend on the group count."""
    with open(os.path.join(GOLDEN, "page_ratios.json")) as f:
        fx = json.load(f)
    sc = fx["lab_scale"]
    table = counts.kv_table(sc["layers"], sc["h"], sc["groups"], sc["seq_len"], sc["head_dim"])
    mha = table[0][1]
    ratios = [mha // e for _, e in table]
    assert [g for g, _ in table] == sc["groups"]
    assert max(ratios) == fx["lab_kv_ratio_max"]
    assert all(mha % e == 0 for _, e in table)
    # the count has no query-head term: 2 * layers * kv_heads * len * head_dim
    assert counts.kv_cache_elems(1, 1, 1, 1) == 2
    assert counts.kv_cache_elems(3, 5, 7, 11) == 2 * 3 * 5 * 7 * 11
    cores = [counts.core_mults(sc["n_tokens"], sc["d_model"], sc["h"], g, sc["head_dim"])
             for g in sc["groups"]]
    assert (len(set(cores)) == 1) == fx["lab_core_same_for_all_g"]
    m8 = counts.mults(sc["n_tokens"], sc["d_model"], sc["h"], 8, sc["head_dim"])
    m1 = counts.mults(sc["n_tokens"], sc["d_model"], sc["h"], 1, sc["head_dim"])
    changed = sorted(k for k in m8 if m8[k] != m1[k] and k != "total")
    assert changed == ["proj_k", "proj_v"]
    assert m8["total"] == sum(v for k, v in m8.items() if k != "total")
    # the multiply ratio stays close to 1 while the cache ratio reaches 8
    assert 1.0 <= m8["total"] / m1["total"] < 1.25
    for key in ("course_llama3_8b", "course_mqa"):
        c = fx[key]
        a = counts.kv_cache_elems(32, c["query_heads"], 8192, 128)
        b = counts.kv_cache_elems(32, c["kv_heads"], 8192, 128)
        assert a // b == c["cache_ratio"] and a % b == 0
    with pytest.raises(ValueError):
        counts.kv_table(32, 8, [3], 4096, 128)
    with pytest.raises(ValueError):
        counts.mults(4096, 1024, 8, 3, 128)


def test_lab_diff_table_first_entry_is_zero(orc):
    """The lab's sample (make_heads(8,6,4, 101/202/303), groups [8,4,2,1]): the first diff_table
    entry is exactly 0.0 and the others are not."""
    import workloads
    q, k, v = (workloads.heads_to_bthd(workloads.make_heads(8, 6, 4, s)) for s in (101, 202, 303))
    ref = orc.heads_out(q, k, v, 8)
    table = [oracle.max_gap(orc.heads_out(q, k, v, g), ref) for g in (8, 4, 2, 1)]
    with open(os.path.join(GOLDEN, "page_ratios.json")) as f:
        assert table[0] == json.load(f)["lab_diff_table_first"]
    assert all(x > 0 for x in table[1:])


def test_generator_logit_statistics():
    """Course step 1: with unit-variance coordinates Var(q.k) = d, so the scaled logits of the
    N(0,1) workloads have mean ~0 and variance ~1."""
    import workloads
    q = workloads.randn_bf16((1, 512, 1, 128), 2000).float().numpy()[0, :, 0].astype(np.float64)
    k = workloads.randn_bf16((1, 512, 1, 128), 2001).float().numpy()[0, :, 0].astype(np.float64)
    s = (q @ k.T) / np.sqrt(128)
    assert abs(s.mean()) < 0.02 and abs(s.var() - 1.0) < 0.05


def test_lcg_is_deterministic_and_bounded():
    import workloads
    a = workloads.make_heads(8, 6, 4, 101)
    b = workloads.make_heads(8, 6, 4, 101)
    assert np.array_equal(a, b) and a.shape == (8, 6, 4)
    assert np.all(np.abs(a) <= 0.5) and not np.array_equal(a, workloads.make_heads(8, 6, 4, 202))
