"""Planted mistakes in the oracle (CPU only): each mutant is a copy of ``gqa_oracle.c`` with one
plausible error, compiled into a temporary library; at least one pin must fail for every mutant.
This shows the pins constrain the oracle and are not a restatement of it."""
import os

import numpy as np
import pytest

import oracle
import oracle_pin_checks as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gqa_oracle.c")

MUTANTS = {
    # step 1: interleaved instead of contiguous groups
    "group_of_interleaved": ("return head / (h / g);", "return head % g;"),
    # step 3: whole-list repetition [A,B,A,B] instead of adjacent repetition
    "expand_tiled": ("&src[((b * T + t) * g + j) * (int64_t)d]",
                     "&src[((b * T + t) * g + (out_head % g)) * (int64_t)d]"),
    # step 2: divide by the head count instead of the group size
    "fold_wrong_divisor": ("dst[((b * T + t) * g + j) * (int64_t)d + c] = acc / (double)s;",
                           "dst[((b * T + t) * g + j) * (int64_t)d + c] = acc / (double)H;"),
    # step 4: scale dropped
    "no_scale": ("s[j] = scale * dot;", "s[j] = dot;"),
    # step 4: max not subtracted
    "no_max_subtraction": ("const double p = exp(s[j] - m);", "const double p = exp(s[j]);"),
    # course step 1: mask one position too strict
    "causal_off_by_one": ("int64_t n = t + (Tkv - Tq) + 1;", "int64_t n = t + (Tkv - Tq);"),
    # top-left instead of bottom-right alignment when Tq < Tkv
    "causal_top_left": ("int64_t n = t + (Tkv - Tq) + 1;", "int64_t n = t + 1;"),
    # softmax not normalised
    "no_normalisation": ("for (int c = 0; c < d; ++c) out[c] /= l;", "(void)l;"),
    # course step 3: window one key too wide
    "window_off_by_one": ("return t + (Tkv - Tq) - window + 1;", "return t + (Tkv - Tq) - window;"),
    # course step 3: sink keys dropped from the window
    "sinks_ignored": ("if (j < lo && j >= n_sink) continue;", "if (j < lo) continue;"),
    # course step 3: rotation turned the wrong way
    "rope_wrong_direction": ("x[2 * i] = re * c - im * s;", "x[2 * i] = re * c + im * s;"),
    # course step 3: query position not aligned with the keys (top-left)
    "rope_query_top_left": ("const int64_t qpos = t + (I.Tkv - I.Tq);", "const int64_t qpos = t;"),
    # backward: replicated key/value heads averaged instead of summed
    "bwd_fold_mean": ("dk[(r * Hkv + j) * (int64_t)d + c] = sk;",
                      "dk[(r * Hkv + j) * (int64_t)d + c] = sk / G;"),
    # backward: softmax Jacobian without the row term D
    "bwd_no_row_term": ("const double ds = p[j] * (dp[j] - D);", "const double ds = p[j] * dp[j];"),
    # backward: query gradient without the scale
    "bwd_dq_no_scale": ("dqr[c] += scale * ds * kh[j * kstride + c];",
                        "dqr[c] += ds * kh[j * kstride + c];"),
    # course step 3: QK-norm with the sum of squares instead of their mean
    "qk_norm_sum_not_mean": ("const double inv = 1.0 / sqrt(ss / d + eps);",
                             "const double inv = 1.0 / sqrt(ss + eps);"),
    # course step 3: QK-norm without its weights
    "qk_norm_no_weights": ("x[c] = x[c] * inv * (double)w[c];", "x[c] = x[c] * inv;"),
    # GVA: every value head of a group reads the group's first value head
    "gva_value_head_of_group": ("const double* vh = &vw[(I.k_row0 * HV + j) * (int64_t)d];",
                                "const double* vh = &vw[(I.k_row0 * HV + j - j % (HV / H)) * "
                                "(int64_t)d];"),
    # selected-rows form: keys left unturned
    "rows_key_rotation_dropped": ("if (rope_mode & ROPE_K) rope_row(&kh[j * d], d, rope_cos, "
                                  "rope_sin, j);", "(void)0;"),
    # selected-rows form: keys turned one position late
    "rows_key_position_shifted": ("rope_row(&kh[j * d], d, rope_cos, rope_sin, j);",
                                  "rope_row(&kh[j * d], d, rope_cos, rope_sin, j + 1);"),
    # selected-rows form: keys not normalised
    "rows_key_norm_dropped": ("if (kn_w) rms_row(&kh[j * d], d, kn_w, norm_eps);", "(void)0;"),
    # value rows weighted by the wrong key
    "value_index_shift": ("out[c] += s[j] * v[j * kstride + c];",
                          "out[c] += s[j] * v[((j + 1) % nvis) * kstride + c];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} no longer in the oracle source"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    import subprocess
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(mutated),
                    "-o", str(lib), "-lm"], check=True)
    orc = oracle.Oracle(str(lib))
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, f"no pin caught mutant {name}"


COUNT_SRC = os.path.join(os.path.dirname(oracle.__file__), "counts.py")

COUNT_MUTANTS = {
    # step 7: projections priced as width x width instead of width x (heads x head dim)
    "proj_width_squared": ('"proj_q": n * d_model * (h * head_dim),',
                           '"proj_q": n * d_model * d_model,'),
    "proj_out_width_squared": ('"proj_out": n * d_model * (h * head_dim),',
                               '"proj_out": n * d_model * d_model,'),
    # step 7: the score term with the group count instead of the query heads
    "scores_use_groups": ('"scores": h * n * n * head_dim,', '"scores": g * n * n * head_dim,'),
    # step 7: value projection with all query heads
    "proj_v_query_heads": ('"proj_v": n * d_model * (g * head_dim),',
                           '"proj_v": n * d_model * (h * head_dim),'),
    # step 6: one tensor instead of K and V
    "cache_one_tensor": ("return 2 * layers * kv_heads * seq_len * head_dim",
                         "return layers * kv_heads * seq_len * head_dim"),
    # step 6: the table indexed by query heads
    "table_query_heads": ("out.append((g, kv_cache_elems(layers, g, seq_len, head_dim)))",
                          "out.append((g, kv_cache_elems(layers, h, seq_len, head_dim)))"),
}


@pytest.mark.parametrize("name", sorted(COUNT_MUTANTS))
def test_count_mutant_is_caught(name):
    import types
    old, new = COUNT_MUTANTS[name]
    src = open(COUNT_SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} no longer in counts.py"
    mod = types.ModuleType("counts_mutant")
    exec(compile(src.replace(old, new), "counts_mutant.py", "exec"), mod.__dict__)
    failed = []
    for check in pins.COUNT_CHECKS:
        try:
            check(mod)
        except (AssertionError, ValueError):
            failed.append(check.__name__)
    assert failed, f"no count pin caught mutant {name}"


# Mistakes in the window-bounded cache's slot rule and visibility (course page "Week 7. Attention",
# step 3), planted in the Python oracle functions for the duration of one check.
WINDOW_CACHE_MUTANTS = {
    # the window's slots start one place late
    "slot_rotated": lambda e, w, s: np.where(e < s, e, s + (e - s + 1) % w),
    # the sinks are not kept apart: every entry cycles through the whole cache
    "slot_ignores_sinks": lambda e, w, s: e % (w + s),
    # the modulo taken from entry 0 instead of from the first non-sink entry
    "slot_from_zero": lambda e, w, s: np.where(e < s, e, s + e % w),
}


@pytest.mark.parametrize("name", sorted(WINDOW_CACHE_MUTANTS))
def test_window_cache_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(oracle, "_window_slots", WINDOW_CACHE_MUTANTS[name])
    orc = oracle.default()
    failed = []
    for check in (pins.check_window_cache_layout, pins.check_window_cache_attention):
        try:
            check(orc)
        except (AssertionError, ValueError, IndexError):
            failed.append(check.__name__)
    assert failed, f"no pin caught window-cache mutant {name}"


def test_window_cache_visibility_mutant_is_caught(monkeypatch):
    """A window one entry too wide."""
    def wide(length, window, n_sink):
        e = np.arange(max(int(length), 0), dtype=np.int64)
        return e[(e < n_sink) | (e >= length - window - 1)]
    monkeypatch.setattr(oracle, "window_cache_visible", wide)
    with pytest.raises(AssertionError):
        pins.check_window_cache_layout(oracle.default())
