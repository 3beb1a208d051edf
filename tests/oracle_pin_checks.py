"""Pins that tie the fp64 oracle to what the pages and the mathematics fix.

Each ``check_*`` function takes a bound oracle (``oracle.Oracle``) and raises AssertionError when
the oracle disagrees with the fact it pins. ``test_oracle_pins.py`` runs them on the in-tree
oracle; ``test_oracle_mutations.py`` runs them on copies of the oracle with a planted mistake and
asserts that some pin fails.

Sources of the facts (page, section):
  * GQA lab page ("Transformer -- attention by hand: reducing only the key/value heads"):
    step 1 (contiguous groups, worked example h=8, g=2), step 2 (fold = mean; g = h returns the
    values unchanged; first-head or global mean only coincide at g = 1), step 3 (expand by
    adjacent repetition, worked example [A,B] -> [A,A,B,B]; query head i reads
    folded[group_of(i)]), step 4 (divide by sqrt(head dim), subtract the max, large inputs must
    not overflow), step 5 (g = h equals multi-head exactly: first diff_table entry 0.0),
    steps 6-8 (counts; cache ratio up to 8x, core multiplies the same for every g).
  * Course page ("Week 7. Attention"): step 1 (scale 1/sqrt(d); -inf before softmax so each row
    still sums to one over the past), step 2 (32/8 heads -> 4x smaller cache, MQA 32x),
    "typical errors" (repeat_kv must repeat adjacently; attention must be causal), and the
    check against torch's scaled_dot_product_attention; step 3 (sliding window and attention
    sinks: the window bounds what a query sees, the first tokens stay visible; rotary position
    embedding: pairs of coordinates turned by pos * theta_i, theta_i = base^(-2i/d), the pair
    being one complex number, so scores depend only on position differences; QK-norm: RMSNorm
    on q and k before the dot product).
  * K3 notes, section 4 (GVA): q and k repeated to the value heads with repeat_interleave
    (forward); the backward of a replication sums over the copies.
"""
from __future__ import annotations

import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa_reference(q, k, v, causal):
    """torch CPU fp64 scaled_dot_product_attention with K/V expanded by repeat_interleave."""
    import torch
    import torch.nn.functional as F
    G = q.shape[2] // k.shape[2]
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64)).permute(0, 2, 1, 3)
    kt = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64)).repeat_interleave(G, dim=2)
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64)).repeat_interleave(G, dim=2)
    kt = kt.permute(0, 2, 1, 3).contiguous()
    vt = vt.permute(0, 2, 1, 3).contiguous()
    out = F.scaled_dot_product_attention(qt.contiguous(), kt, vt, is_causal=causal)
    return out.permute(0, 2, 1, 3).numpy()


# ------------------------------------------------------------------------------------------------
# step 1: grouping
# ------------------------------------------------------------------------------------------------

def check_group_of_worked_example(orc):
    with open(os.path.join(GOLDEN, "group_map_h8_g2.txt")) as f:
        rows = [tuple(int(x) for x in ln.split()) for ln in f
                if ln.strip() and not ln.startswith("#")]
    assert rows, "fixture empty"
    for h, g, head, grp in rows:
        assert orc.group_of(head, h, g) == grp, (h, g, head)
    # contiguous blocks: group sizes equal, each group a run of consecutive heads
    for h in range(1, 9):
        for g in [x for x in range(1, h + 1) if h % x == 0]:
            mem = orc.group_members(h, g)
            assert [x for grp in mem for x in grp] == list(range(h)), (h, g)
            assert all(len(grp) == h // g for grp in mem)


def check_group_of_rejects_uneven(orc):
    for h, g in ((8, 3), (6, 4), (32, 5)):
        try:
            orc.group_members(h, g)
        except ValueError:
            continue
        raise AssertionError(f"group_members({h},{g}) did not raise")


# ------------------------------------------------------------------------------------------------
# step 2: fold
# ------------------------------------------------------------------------------------------------

def check_fold_identity_when_g_is_h(orc):
    x = _rng(1).standard_normal((2, 5, 8, 16)).astype(np.float32)
    f = orc.fold_kv(x, 8)
    assert np.array_equal(f, x.astype(np.float64))


def check_fold_is_group_mean(orc):
    # integer-valued inputs: every sum and the division by a power of two are exact
    x = _rng(2).integers(-64, 64, size=(2, 3, 8, 4)).astype(np.float64)
    for g in (4, 2, 1):
        s = 8 // g
        want = x.reshape(2, 3, g, s, 4).sum(axis=3) / s
        assert np.array_equal(orc.fold_kv(x, g), want), g
    # constant within each group -> that constant
    c = np.repeat(np.arange(4.0)[None, None, :, None], 2, axis=2).reshape(1, 1, 8, 1)
    c = np.broadcast_to(c, (1, 2, 8, 3)).copy()
    assert np.array_equal(orc.fold_kv(c, 4), np.broadcast_to(np.arange(4.0)[None, None, :, None],
                                                              (1, 2, 4, 3)))
    # the lab: keeping the first head, or averaging everything, only agree with fold at g = 1
    y = _rng(3).standard_normal((1, 4, 8, 4))
    f2 = orc.fold_kv(y, 2)
    assert not np.allclose(f2[:, :, 0], y[:, :, 0])
    assert not np.allclose(f2[:, :, 0], y.mean(axis=2))
    assert np.allclose(orc.fold_kv(y, 1)[:, :, 0], y.mean(axis=2), rtol=0, atol=1e-15)


# ------------------------------------------------------------------------------------------------
# step 3: expand
# ------------------------------------------------------------------------------------------------

def check_expand_worked_example(orc):
    with open(os.path.join(GOLDEN, "expand_AB_to_4.txt")) as f:
        line = [ln for ln in f if ln.strip() and not ln.startswith("#")][0]
    src, h, want, wrong = [p.strip() for p in line.split("|")]
    names = src.split(",")
    h = int(h)
    folded = np.arange(1.0, len(names) + 1.0).reshape(1, 1, len(names), 1)  # A=1, B=2
    code = {n: float(i + 1) for i, n in enumerate(names)}
    got = orc.expand_kv(folded, h)[0, 0, :, 0]
    assert list(got) == [code[n] for n in want.split(",")]
    assert list(got) != [code[n] for n in wrong.split(",")]


def check_expand_reads_own_group(orc):
    x = _rng(4).standard_normal((1, 3, 8, 5))
    for g in (8, 4, 2, 1):
        f = orc.fold_kv(x, g)
        e = orc.expand_kv(f, 8)
        members = orc.group_members(8, g)
        for i in range(8):
            gi = orc.group_of(i, 8, g)
            assert np.array_equal(e[:, :, i], f[:, :, gi]), (g, i)
            assert np.allclose(e[:, :, i], x[:, :, members[gi]].mean(axis=2), rtol=0, atol=1e-14)


# ------------------------------------------------------------------------------------------------
# step 4 / course step 1: attention
# ------------------------------------------------------------------------------------------------

def check_matches_torch_sdpa(orc):
    """Library cross-check: every divisor Hkv of Hq <= 8, unmasked and square causal, plus a
    bottom-right-free decode case (Tq = 1, unmasked)."""
    rng = _rng(5)
    for Hq in (1, 2, 3, 4, 6, 8):
        for Hkv in [x for x in range(1, Hq + 1) if Hq % x == 0]:
            for causal in (False, True):
                q = rng.standard_normal((2, 7, Hq, 8))
                k = rng.standard_normal((2, 7, Hkv, 8))
                v = rng.standard_normal((2, 7, Hkv, 8))
                got = orc.attention(q, k, v, causal=causal)
                ref = _sdpa_reference(q, k, v, causal)
                err = np.max(np.abs(got - ref))
                assert err <= 1e-12, (Hq, Hkv, causal, err)
    q = rng.standard_normal((3, 1, 8, 16))
    k = rng.standard_normal((3, 33, 2, 16))
    v = rng.standard_normal((3, 33, 2, 16))
    assert np.max(np.abs(orc.attention(q, k, v) - _sdpa_reference(q, k, v, False))) <= 1e-12


def check_scale_is_one_over_sqrt_d(orc):
    # d = 16 -> scale 1/4. q = 4a e_0, k_1 = b e_0 with a*b = ln 3: scores 0 and ln 3, weights 1/4, 3/4
    d = 16
    q = np.zeros((1, 1, 1, d)); q[0, 0, 0, 0] = 4.0
    k = np.zeros((1, 2, 1, d)); k[0, 1, 0, 0] = math.log(3.0)
    v = np.zeros((1, 2, 1, d)); v[0, 0, 0, :] = 1.0; v[0, 1, 0, :] = 5.0
    out = orc.attention(q, k, v)
    assert np.allclose(out, 0.25 * 1.0 + 0.75 * 5.0, rtol=0, atol=1e-14), out[0, 0, 0, 0]
    # default scale equals an explicit 1/sqrt(d)
    x = _rng(6).standard_normal((1, 9, 2, d))
    assert np.array_equal(orc.attention(x, x[:, :, :1], x[:, :, 1:]),
                          orc.attention(x, x[:, :, :1], x[:, :, 1:], scale=0.25))


def check_rows_sum_to_one(orc):
    # V rows = unit basis vectors: the output row is the softmax weight vector itself
    rng = _rng(7)
    T, d = 12, 16
    q = rng.standard_normal((1, T, 4, d)) * 3
    k = rng.standard_normal((1, T, 2, d)) * 3
    v = np.zeros((1, T, 2, d)); v[0, np.arange(T), :, np.arange(T)] = 1.0
    for causal in (False, True):
        w = orc.attention(q, k, v, causal=causal)
        assert np.all(w >= 0)
        assert np.allclose(w.sum(axis=-1), 1.0, rtol=0, atol=1e-14)
        if causal:  # nothing after the query's own position
            for t in range(T):
                assert np.all(w[0, t, :, t + 1:T] == 0.0)


def check_closed_forms(orc):
    rng = _rng(8)
    # V == 1 -> out == 1
    q = rng.standard_normal((2, 6, 4, 8)); k = rng.standard_normal((2, 6, 2, 8))
    assert np.allclose(orc.attention(q, k, np.ones((2, 6, 2, 8)), causal=True), 1.0, rtol=0,
                       atol=1e-15)
    # K == 0 -> uniform weights: prefix means (causal) or full mean (unmasked)
    v = rng.standard_normal((1, 6, 2, 8))
    z = np.zeros((1, 6, 2, 8)); q1 = rng.standard_normal((1, 6, 4, 8))
    o_full = orc.attention(q1, z, v)
    o_causal = orc.attention(q1, z, v, causal=True)
    for i in range(4):
        kv = i // 2
        assert np.allclose(o_full[0, :, i], v[0, :, kv].mean(axis=0), rtol=0, atol=1e-14)
        for t in range(6):
            assert np.allclose(o_causal[0, t, i], v[0, :t + 1, kv].mean(axis=0), rtol=0,
                               atol=1e-14)
    # a single key -> out == v_0 exactly
    v1 = rng.standard_normal((1, 1, 1, 8))
    assert np.array_equal(orc.attention(rng.standard_normal((1, 3, 4, 8)),
                                        rng.standard_normal((1, 1, 1, 8)), v1)[0, :, 0],
                          np.repeat(v1[0, :, 0], 3, axis=0))
    # one dominant key -> its value row
    k2 = rng.standard_normal((1, 5, 1, 8)) * 0.1
    qd = np.zeros((1, 1, 1, 8)); qd[0, 0, 0, 0] = 100.0
    k2[0, 3, 0, 0] = 100.0
    assert np.allclose(orc.attention(qd, k2, v[:, :5, :1])[0, 0, 0], v[0, 3, 0], rtol=0,
                       atol=1e-12)


def check_large_inputs_do_not_overflow(orc):
    rng = _rng(9)
    for mult in (1e3, 1e6):
        q = rng.standard_normal((1, 8, 4, 16)) * mult
        k = rng.standard_normal((1, 8, 2, 16)) * mult
        v = rng.standard_normal((1, 8, 2, 16))
        out = orc.attention(q, k, v, causal=True)
        assert np.all(np.isfinite(out))
        # at this scale every row is one-hot on its best visible key
        G = 2
        for t in range(8):
            for i in range(4):
                s = [float(q[0, t, i] @ k[0, j, i // G]) for j in range(t + 1)]
                assert np.allclose(out[0, t, i], v[0, int(np.argmax(s)), i // G], rtol=0,
                                   atol=1e-9)


def check_causality(orc):
    rng = _rng(10)
    q = rng.standard_normal((1, 10, 4, 8)); k = rng.standard_normal((1, 10, 2, 8))
    v = rng.standard_normal((1, 10, 2, 8))
    base = orc.attention(q, k, v, causal=True)
    for t in (0, 4, 8):
        k2 = k.copy(); v2 = v.copy()
        k2[0, t + 1:] += 7.0; v2[0, t + 1:] -= 3.0
        o = orc.attention(q, k2, v2, causal=True)
        assert np.array_equal(o[0, :t + 1], base[0, :t + 1]), t
        assert not np.array_equal(o[0, t + 1:], base[0, t + 1:]), t


def check_bottom_right_alignment(orc):
    """Tq < Tkv with the causal flag equals the last Tq rows of square causal attention over Tkv
    queries (square causal is pinned to torch above); a single query sees the whole cache."""
    rng = _rng(11)
    Tkv, Tq = 11, 4
    qf = rng.standard_normal((2, Tkv, 4, 8))
    k = rng.standard_normal((2, Tkv, 1, 8)); v = rng.standard_normal((2, Tkv, 1, 8))
    full = orc.attention(qf, k, v, causal=True)
    part = orc.attention(qf[:, Tkv - Tq:], k, v, causal=True)
    assert np.array_equal(part, full[:, Tkv - Tq:])
    one = orc.attention(qf[:, -1:], k, v, causal=True)
    assert np.array_equal(one, orc.attention(qf[:, -1:], k, v, causal=False))


# ------------------------------------------------------------------------------------------------
# step 5: heads_out / max_gap
# ------------------------------------------------------------------------------------------------

def check_g_equals_h_is_mha(orc):
    from oracle import max_gap
    q = _rng(12).standard_normal((1, 6, 8, 4))
    k = _rng(13).standard_normal((1, 6, 8, 4))
    v = _rng(14).standard_normal((1, 6, 8, 4))
    mha = np.concatenate([orc.attention(q[:, :, i:i + 1], k[:, :, i:i + 1], v[:, :, i:i + 1])
                          for i in range(8)], axis=2)
    gaps = [max_gap(orc.heads_out(q, k, v, g), mha) for g in (8, 4, 2, 1)]
    assert gaps[0] == 0.0, gaps
    assert all(gp > 0 for gp in gaps[1:]), gaps


def check_packed_equals_separate(orc):
    rng = _rng(15)
    lens = (5, 1, 9, 3)
    tot = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = rng.standard_normal((1, tot, 4, 8)); k = rng.standard_normal((1, tot, 2, 8))
    v = rng.standard_normal((1, tot, 2, 8))
    packed = orc.attention(q, k, v, causal=True, cu_seqlens=cu)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        sep = orc.attention(q[:, a:b], k[:, a:b], v[:, a:b], causal=True)
        assert np.array_equal(packed[:, a:b], sep), s


def check_rows_equal_full(orc):
    rng = _rng(16)
    q = rng.standard_normal((2, 9, 8, 8)).astype(np.float32)
    k = rng.standard_normal((2, 9, 2, 8)).astype(np.float32)
    v = rng.standard_normal((2, 9, 2, 8)).astype(np.float32)
    full = orc.attention(q, k, v, causal=True)
    rows = np.array([(0, 0, 0), (1, 8, 7), (1, 3, 2), (0, 5, 5)], dtype=np.int64)
    got = orc.attention_rows(q, k, v, rows, causal=True)
    for r, (b, t, h) in enumerate(rows):
        assert np.array_equal(got[r], full[b, t, h]), (b, t, h)
    cu = np.array([0, 3, 9], dtype=np.int32)
    qp, kp, vp = q[:1], k[:1], v[:1]
    fullp = orc.attention(qp, kp, vp, causal=True, cu_seqlens=cu)
    rows = np.array([(0, 0, 1), (0, 2, 7), (0, 3, 0), (0, 8, 4)], dtype=np.int64)
    got = orc.attention_rows(qp, kp, vp, rows, causal=True, cu_seqlens=cu)
    for r, (b, t, h) in enumerate(rows):
        assert np.array_equal(got[r], fullp[b, t, h]), (b, t, h)


def _torch_prepared_sdpa(q, k, v, causal, tabs=None, norm=None, keys_done=False):
    """torch fp64 reference of attention with QK-norm (torch rms_norm) and then the rotary turn
    (complex multiplication) applied to q and, unless ``keys_done``, to k; query t at position
    t + Tkv - Tq, key j at position j (course page, step 3). Dense batch; numpy out."""
    import torch
    import torch.nn.functional as F
    d = q.shape[3]
    Tq, Tkv = q.shape[1], k.shape[1]

    def norm_rows(x, w):
        return F.rms_norm(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)), (d,),
                          torch.from_numpy(w.astype(np.float64)), norm[2])

    def turn(x, pos0):
        if tabs is None:
            return x
        rot = torch.complex(torch.from_numpy(tabs[0].astype(np.float64)),
                            torch.from_numpy(tabs[1].astype(np.float64)))
        z = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous())
        z = z * rot[pos0:pos0 + x.shape[1]][None, :, None, :]
        return torch.view_as_real(z).reshape(x.shape)
    qq = norm_rows(q, norm[0]) if norm is not None else torch.from_numpy(np.float64(q))
    kk = torch.from_numpy(np.float64(k))
    if not keys_done:
        kk = norm_rows(k, norm[1]) if norm is not None else kk
        kk = turn(kk, 0)
    G = q.shape[2] // k.shape[2]
    qt = turn(qq, Tkv - Tq).permute(0, 2, 1, 3).contiguous()
    kt = kk.repeat_interleave(G, dim=2).permute(0, 2, 1, 3).contiguous()
    vt = torch.from_numpy(np.float64(v)).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    mask = torch.from_numpy(_window_mask(Tq, Tkv, Tkv + 1, 0)) if causal else None
    ref = F.scaled_dot_product_attention(qt, kt, vt.contiguous(), attn_mask=mask)
    return ref.permute(0, 2, 1, 3).numpy()


def check_rows_with_rope_and_norm(orc):
    """The selected-rows form with the course page's step-3 prologues (rotary turn from
    position tables, QK-norm with caller weights, both together), with fewer queries than keys
    (query t at position t + Tkv - Tq) and in packed batches (positions per sequence): each row
    equals the whole-output oracle exactly and torch's rms_norm + complex rotation + fp64 SDPA
    to 1e-12."""
    rng = _rng(29)
    d, Hq, Hkv = 8, 6, 2
    cases = [(5, 9, True, "qk", False), (7, 7, True, "qk", True), (4, 9, True, None, True),
             (3, 10, False, "qk", True), (6, 6, True, "q", False), (4, 8, True, "q", True)]
    for Tq, Tkv, causal, rope_mode, use_norm in cases:
        q = rng.standard_normal((2, Tq, Hq, d)) * 2.0
        k = rng.standard_normal((2, Tkv, Hkv, d))
        v = rng.standard_normal((2, Tkv, Hkv, d))
        tabs = rope_tables(Tkv + 3, d) if rope_mode else None
        norm = None
        if use_norm:
            norm = ((rng.random(d) + 0.5).astype(np.float32),
                    (rng.random(d) + 0.5).astype(np.float32), 1e-6)
        keys_done = rope_mode == "q"
        kin = k
        if keys_done:
            # a cache: keys normalised and turned beforehand, by torch
            kin = _torch_prepared_sdpa_keys(k, tabs, norm)
        kw = dict(causal=causal, rope=tabs, rope_mode=rope_mode or "qk", qk_norm=norm,
                  qk_norm_mode="q" if keys_done else "qk")
        full = orc.attention(q, kin, v, **kw)
        rows = np.array([(0, 0, 0), (1, Tq - 1, Hq - 1), (1, Tq // 2, 2), (0, Tq - 1, 3),
                         (1, 0, 5)], dtype=np.int64)
        got = orc.attention_rows(q, kin, v, rows, **kw)
        ref = _torch_prepared_sdpa(q, kin, v, causal, tabs, norm, keys_done)
        for r, (b, t, h) in enumerate(rows):
            assert np.array_equal(got[r], full[b, t, h]), (Tq, Tkv, rope_mode, use_norm, b, t, h)
            err = np.max(np.abs(got[r] - ref[b, t, h]))
            assert err <= 1e-12, (Tq, Tkv, rope_mode, use_norm, b, t, h, err)
    # packed: two sequences of 4 and 7 tokens, each turned from its own position 0
    cu = np.array([0, 4, 11], dtype=np.int32)
    q = rng.standard_normal((1, 11, Hq, d)); k = rng.standard_normal((1, 11, Hkv, d))
    v = rng.standard_normal((1, 11, Hkv, d))
    tabs = rope_tables(8, d)
    norm = ((rng.random(d) + 0.5).astype(np.float32), (rng.random(d) + 0.5).astype(np.float32),
            1e-5)
    kw = dict(causal=True, cu_seqlens=cu, rope=tabs, qk_norm=norm)
    full = orc.attention(q, k, v, **kw)
    rows = np.array([(0, 0, 0), (0, 3, 5), (0, 4, 1), (0, 10, 4), (0, 7, 2)], dtype=np.int64)
    got = orc.attention_rows(q, k, v, rows, **kw)
    for s in range(2):
        a, b = int(cu[s]), int(cu[s + 1])
        ref = _torch_prepared_sdpa(q[:, a:b], k[:, a:b], v[:, a:b], True, tabs, norm)
        for r, (_, t, h) in enumerate(rows):
            if a <= t < b:
                assert np.array_equal(got[r], full[0, t, h]), (t, h)
                assert np.max(np.abs(got[r] - ref[0, t - a, h])) <= 1e-12, (t, h)


def _torch_prepared_sdpa_keys(k, tabs, norm):
    """Keys normalised (torch rms_norm) and turned (complex multiplication) at positions 0.."""
    import torch
    import torch.nn.functional as F
    d = k.shape[3]
    kk = torch.from_numpy(np.float64(k))
    if norm is not None:
        kk = F.rms_norm(kk, (d,), torch.from_numpy(norm[1].astype(np.float64)), norm[2])
    if tabs is not None:
        rot = torch.complex(torch.from_numpy(tabs[0].astype(np.float64)),
                            torch.from_numpy(tabs[1].astype(np.float64)))
        z = torch.view_as_complex(kk.reshape(*kk.shape[:-1], d // 2, 2).contiguous())
        z = z * rot[0:kk.shape[1]][None, :, None, :]
        kk = torch.view_as_real(z).reshape(kk.shape)
    return kk.numpy()


def check_bf16_widening_is_exact(orc):
    bits = _rng(17).integers(0, 1 << 16, size=(1, 5, 4, 8), dtype=np.uint16)
    bits[(bits & 0x7F80) == 0x7F80] = 0x3F80    # no inf/nan patterns
    vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    vals = np.clip(vals, -1e3, 1e3)
    bits = ((vals.astype(np.float32)).view(np.uint32) >> 16).astype(np.uint16)
    vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    kb, vb = bits[:, :, :2], bits[:, :, 2:]
    a = orc.attention(bits, np.ascontiguousarray(kb), np.ascontiguousarray(vb), causal=True)
    b = orc.attention(vals, vals[:, :, :2], vals[:, :, 2:], causal=True)
    assert np.array_equal(a, b)


# ------------------------------------------------------------------------------------------------
# course step 3: sliding window and attention sinks
# ------------------------------------------------------------------------------------------------

def _window_mask(Tq, Tkv, window, n_sink):
    """Boolean [Tq, Tkv] table built from the definition: query t sits at p = t + Tkv - Tq and
    sees key j iff j <= p and (j > p - window or j < n_sink)."""
    m = np.zeros((Tq, Tkv), dtype=bool)
    for t in range(Tq):
        p = t + Tkv - Tq
        for j in range(Tkv):
            m[t, j] = j <= p and (j > p - window or j < n_sink)
    return m


def check_window_matches_masked_sdpa(orc):
    """Library cross-check: torch CPU fp64 scaled_dot_product_attention with an explicit mask
    table (K/V expanded by repeat_interleave), for windows with and without sink keys."""
    import torch
    import torch.nn.functional as F
    rng = _rng(18)
    for (Tq, Tkv, W, S) in [(9, 9, 3, 0), (9, 9, 3, 2), (5, 12, 4, 1), (12, 12, 1, 3),
                            (7, 7, 20, 0), (1, 30, 8, 4), (16, 16, 5, 5)]:
        for Hq, Hkv in ((4, 2), (3, 1), (2, 2)):
            q = rng.standard_normal((2, Tq, Hq, 8))
            k = rng.standard_normal((2, Tkv, Hkv, 8))
            v = rng.standard_normal((2, Tkv, Hkv, 8))
            got = orc.attention(q, k, v, causal=True, window=W, n_sink=S)
            G = Hq // Hkv
            qt = torch.from_numpy(q).permute(0, 2, 1, 3).contiguous()
            kt = torch.from_numpy(k).repeat_interleave(G, dim=2).permute(0, 2, 1, 3).contiguous()
            vt = torch.from_numpy(v).repeat_interleave(G, dim=2).permute(0, 2, 1, 3).contiguous()
            mask = torch.from_numpy(_window_mask(Tq, Tkv, W, S))
            ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
            err = np.max(np.abs(got - ref.permute(0, 2, 1, 3).numpy()))
            assert err <= 1e-12, (Tq, Tkv, W, S, Hq, Hkv, err)


def check_window_limits(orc):
    """A window covering the whole past (or sinks covering it) is plain causal attention; a
    one-key window returns each query's own value row; windows need the causal flag."""
    rng = _rng(19)
    q = rng.standard_normal((2, 6, 4, 8)); k = rng.standard_normal((2, 10, 2, 8))
    v = rng.standard_normal((2, 10, 2, 8))
    causal = orc.attention(q, k, v, causal=True)
    assert np.array_equal(orc.attention(q, k, v, causal=True, window=10), causal)
    assert np.array_equal(orc.attention(q, k, v, causal=True, window=3, n_sink=10), causal)
    one = orc.attention(q, k, v, causal=True, window=1)
    for t in range(6):
        for h in range(4):
            assert np.array_equal(one[:, t, h], v[:, t + 4, h // 2]), (t, h)
    rows = np.array([(0, 0, 0), (1, 5, 3), (0, 3, 2)], dtype=np.int64)
    full = orc.attention(q, k, v, causal=True, window=3, n_sink=2)
    got = orc.attention_rows(q, k, v, rows, causal=True, window=3, n_sink=2)
    for r, (b, t, h) in enumerate(rows):
        assert np.array_equal(got[r], full[b, t, h]), (b, t, h)
    try:
        orc.attention(q, k, v, causal=False, window=3)
    except ValueError:
        pass
    else:
        raise AssertionError("a window without the causal flag must be rejected")


def _fill_window_cache(k, window, n_sink):
    """Writes the entries of a full cache k [B, L, ...] one at a time into a cache bounded to the
    window, the way a decoder fills it: the first n_sink entries into their own slots, then a
    cursor that steps through the window's slots and starts over at the first of them when it
    passes the last; a first-in-first-out queue of at most `window` entries records which
    entries the bounded cache should still hold. Returns the cache and the queue's entries plus
    the sinks. Shares nothing with the oracle's closed-form slot rule."""
    from collections import deque
    B, L = k.shape[:2]
    ring = np.zeros((B, n_sink + window) + k.shape[2:], dtype=k.dtype)
    held = np.full(n_sink + window, -1)
    fifo = deque(maxlen=window)
    cur = n_sink
    for e in range(L):
        if e < n_sink:
            slot = e
        else:
            slot = cur
            cur = cur + 1 if cur + 1 < n_sink + window else n_sink
            fifo.append(e)
        ring[:, slot] = k[:, e]
        held[slot] = e
    kept = sorted(list(range(min(L, n_sink))) + list(fifo))
    return ring, held, kept


def check_window_cache_layout(orc):
    """The bounded cache's layout: after a writer fills it entry by entry (cursor and queue, above),
    the entries it holds are exactly the ones a windowed query at the last position sees (course
    step 3: the window bounds the cache, the sinks stay), each at the slot the oracle reads it
    from; for every window, sink count and length up to three times the capacity."""
    del orc
    for W, S in [(1, 0), (1, 3), (4, 0), (4, 2), (7, 5), (16, 1), (3, 9)]:
        for L in range(0, 3 * (W + S) + 5):
            _, held, kept = _fill_window_cache(np.arange(L).reshape(1, L), W, S)
            vis = oracle.window_cache_visible(L, W, S)
            assert list(vis) == kept, (W, S, L, list(vis), kept)
            assert sorted(int(x) for x in held if x >= 0) == kept, (W, S, L)
            for e in vis:
                assert held[oracle.window_cache_slot(int(e), W, S)] == e, (W, S, L, e)


def check_window_cache_attention(orc):
    """Decode from a bounded cache equals the windowed decode of the full cache bit for bit,
    unrolled (hidden entries zero) and compact (visible entries only, no window), for plain,
    rotary (query turned at the last position, keys turned when written) and QK-norm queries."""
    rng = _rng(31)
    for (L, W, S, Hq, Hkv) in [(1, 4, 0, 4, 2), (3, 4, 2, 4, 2), (6, 4, 2, 4, 1), (23, 5, 3, 6, 3),
                               (40, 7, 0, 2, 2), (40, 1, 1, 4, 2), (9, 16, 4, 4, 2)]:
        d = 8
        q = rng.standard_normal((1, 1, Hq, d))
        k = rng.standard_normal((1, L, Hkv, d))
        v = rng.standard_normal((1, L, Hkv, d))
        rk, _, _ = _fill_window_cache(k, W, S)
        rv, _, _ = _fill_window_cache(v, W, S)
        ref = orc.attention(q, k, v, causal=True, window=W, n_sink=S)
        ku = oracle.unroll_window_cache(rk, [L], W, S)[0]
        vu = oracle.unroll_window_cache(rv, [L], W, S)[0]
        assert np.array_equal(orc.attention(q, ku, vu, causal=True, window=W, n_sink=S), ref)
        kc = oracle.unroll_window_cache(rk, [L], W, S, compact=True)[0]
        vc = oracle.unroll_window_cache(rv, [L], W, S, compact=True)[0]
        assert kc.shape[1] == min(L, W + S)
        assert np.array_equal(orc.attention(q, kc, vc), ref), (L, W, S)
        cos, sin = rope_tables(L, d)
        rref = orc.attention(q, k, v, causal=True, window=W, n_sink=S, rope=(cos, sin),
                             rope_mode="q")
        assert np.array_equal(orc.attention(q, ku, vu, causal=True, window=W, n_sink=S,
                                            rope=(cos, sin), rope_mode="q"), rref)
        norm = (rng.standard_normal(d).astype(np.float32), np.ones(d, dtype=np.float32), 1e-6)
        nref = orc.attention(q, k, v, causal=True, window=W, n_sink=S, qk_norm=norm,
                             qk_norm_mode="q")
        assert np.array_equal(orc.attention(q, ku, vu, causal=True, window=W, n_sink=S,
                                            qk_norm=norm, qk_norm_mode="q"), nref)


# ------------------------------------------------------------------------------------------------
# course step 3: rotary position embedding
# ------------------------------------------------------------------------------------------------

def rope_tables(npos, d, base=10000.0):
    """cos / sin of p * theta_i with theta_i = base^(-2i/d), computed in float64 and stored as
    float32 [npos, d/2] (the course page's formula, step 3)."""
    i = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / d)
    ang = np.arange(npos, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def check_rope_worked_example(orc):
    """d = 2 (theta_0 = 1 rad per position): q = (1, 0) at position 1 turns to (cos 1, sin 1);
    key 0 = (0, 1) stays, key 1 = (1, 0) turns with q. Scores sin(1)/sqrt(2) and 1/sqrt(2), so
    out = softmax-weighted v0 = (1, 0), v1 = (0, 1) in closed form. A turn in the other direction
    would give the first score the opposite sign."""
    cos_t, sin_t = rope_tables(2, 2)
    q = np.array([1.0, 0.0]).reshape(1, 1, 1, 2)
    k = np.array([[0.0, 1.0], [1.0, 0.0]]).reshape(1, 2, 1, 2)
    v = np.array([[1.0, 0.0], [0.0, 1.0]]).reshape(1, 2, 1, 2)
    got = orc.attention(q, k, v, causal=True, rope=(cos_t, sin_t))
    c1, s1 = float(cos_t[1, 0]), float(sin_t[1, 0])
    sc = 1.0 / math.sqrt(2.0)
    s0v, s1v = sc * s1, sc * (c1 * c1 + s1 * s1)
    p0 = 1.0 / (1.0 + math.exp(s1v - s0v))
    assert abs(got[0, 0, 0, 0] - p0) <= 1e-14 and abs(got[0, 0, 0, 1] - (1 - p0)) <= 1e-14, got


def check_rope_matches_complex_torch(orc):
    """Library cross-check: rotate q and k by complex multiplication in torch (the page's complex
    form: adjacent coordinates are the real and imaginary part), then torch fp64 SDPA."""
    import torch
    import torch.nn.functional as F
    rng = _rng(20)
    for (Tq, Tkv, Hq, Hkv, d, causal) in [(7, 7, 4, 2, 8, True), (3, 11, 2, 1, 16, True),
                                          (5, 5, 3, 3, 4, False)]:
        cos_t, sin_t = rope_tables(Tkv + 2, d)
        q = rng.standard_normal((2, Tq, Hq, d)); k = rng.standard_normal((2, Tkv, Hkv, d))
        v = rng.standard_normal((2, Tkv, Hkv, d))
        got = orc.attention(q, k, v, causal=causal, rope=(cos_t, sin_t))
        rot = torch.complex(torch.from_numpy(cos_t.astype(np.float64)),
                            torch.from_numpy(sin_t.astype(np.float64)))

        def turn(x, pos0):
            z = torch.view_as_complex(torch.from_numpy(x).reshape(*x.shape[:-1], d // 2, 2))
            z = z * rot[pos0:pos0 + x.shape[1]][None, :, None, :]
            return torch.view_as_real(z).reshape(x.shape)
        G = Hq // Hkv
        qt = turn(q, Tkv - Tq).permute(0, 2, 1, 3).contiguous()
        kt = turn(k, 0).repeat_interleave(G, dim=2).permute(0, 2, 1, 3).contiguous()
        vt = torch.from_numpy(v).repeat_interleave(G, dim=2).permute(0, 2, 1, 3).contiguous()
        mask = None
        if causal:
            mask = torch.from_numpy(_window_mask(Tq, Tkv, Tkv + 1, 0))
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
        err = np.max(np.abs(got - ref.permute(0, 2, 1, 3).numpy()))
        assert err <= 1e-12, (Tq, Tkv, d, causal, err)
        # queries only (keys already turned, as in a cache)
        k_turned = turn(k, 0).numpy()
        got_q = orc.attention(q, k_turned, v, causal=causal, rope=(cos_t, sin_t), rope_mode="q")
        assert np.max(np.abs(got_q - got)) <= 1e-12


def check_rope_relative_positions(orc):
    """Scores depend on positions only through m - n (the page's derivation): moving every
    position by the same amount (tables read from a later row) leaves the output unchanged up
    to the fp32 rounding of the tables; zero angles are no rotation at all."""
    rng = _rng(21)
    d = 16
    cos_t, sin_t = rope_tables(64, d)
    q = rng.standard_normal((1, 9, 4, d)); k = rng.standard_normal((1, 9, 2, d))
    v = rng.standard_normal((1, 9, 2, d))
    a = orc.attention(q, k, v, causal=True, rope=(cos_t, sin_t))
    b = orc.attention(q, k, v, causal=True, rope=(cos_t[37:], sin_t[37:]))
    assert np.max(np.abs(a - b)) <= 1e-5, np.max(np.abs(a - b))
    assert np.max(np.abs(a - orc.attention(q, k, v, causal=True))) > 1e-3
    ones, zeros = np.ones_like(cos_t), np.zeros_like(sin_t)
    assert np.array_equal(orc.attention(q, k, v, causal=True, rope=(ones, zeros)),
                          orc.attention(q, k, v, causal=True))


def check_qk_norm_matches_torch_rms_norm(orc):
    """Library cross-check of QK-norm (course page, step 3: RMSNorm on q and k before the dot
    product): torch's rms_norm over the head dim with the same weights and eps, then the rotation
    (complex multiplication), then fp64 SDPA; and the queries-only form against pre-processed
    keys (a cache)."""
    import torch
    import torch.nn.functional as F
    rng = _rng(27)
    for (Tq, Tkv, Hq, Hkv, d, causal, rope) in [(6, 6, 4, 2, 8, True, False),
                                                (4, 9, 3, 1, 16, True, True),
                                                (5, 5, 2, 2, 8, False, True)]:
        q = rng.standard_normal((2, Tq, Hq, d)) * 3.0
        k = rng.standard_normal((2, Tkv, Hkv, d)) * 0.5
        v = rng.standard_normal((2, Tkv, Hkv, d))
        wq = (rng.random(d) + 0.5).astype(np.float32)
        wk = (rng.random(d) + 0.5).astype(np.float32)
        eps = 1e-6
        tabs = rope_tables(Tkv + 1, d) if rope else None
        got = orc.attention(q, k, v, causal=causal, rope=tabs, qk_norm=(wq, wk, eps))

        def norm(x, w):
            return F.rms_norm(torch.from_numpy(x), (d,), torch.from_numpy(w.astype(np.float64)),
                              eps)

        def turn(x, pos0):
            if not rope:
                return x
            rot = torch.complex(torch.from_numpy(tabs[0].astype(np.float64)),
                                torch.from_numpy(tabs[1].astype(np.float64)))
            z = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous())
            z = z * rot[pos0:pos0 + x.shape[1]][None, :, None, :]
            return torch.view_as_real(z).reshape(x.shape)
        G = Hq // Hkv
        qt = turn(norm(q, wq), Tkv - Tq).permute(0, 2, 1, 3).contiguous()
        kp = turn(norm(k, wk), 0)
        kt = kp.repeat_interleave(G, dim=2).permute(0, 2, 1, 3).contiguous()
        vt = torch.from_numpy(v).repeat_interleave(G, dim=2).permute(0, 2, 1, 3).contiguous()
        mask = torch.from_numpy(_window_mask(Tq, Tkv, Tkv + 1, 0)) if causal else None
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
        err = np.max(np.abs(got - ref.permute(0, 2, 1, 3).numpy()))
        assert err <= 1e-12, (Tq, Tkv, d, causal, rope, err)
        got_q = orc.attention(q, kp.numpy(), v, causal=causal, rope=tabs, rope_mode="q",
                              qk_norm=(wq, wk, eps), qk_norm_mode="q")
        assert np.max(np.abs(got_q - got)) <= 1e-12


def check_qk_norm_worked_example_and_scale_invariance(orc):
    """d = 2, unit weights, eps = 0: q = (3, 4) normalises to (3, 4) / sqrt(12.5); keys (1, 0) and
    (0, 2) to (sqrt 2, 0) and (0, sqrt 2); the two scores and the output follow in closed form.
    And with eps = 0 the output does not change when q or k is scaled by a positive factor (the
    point of the norm: it fixes the scale of the logits)."""
    q = np.array([3.0, 4.0]).reshape(1, 1, 1, 2)
    k = np.array([[1.0, 0.0], [0.0, 2.0]]).reshape(1, 2, 1, 2)
    v = np.array([[1.0, 0.0], [0.0, 1.0]]).reshape(1, 2, 1, 2)
    one = np.ones(2, dtype=np.float32)
    got = orc.attention(q, k, v, qk_norm=(one, one, 0.0))
    r = math.sqrt(12.5)
    s0 = (3.0 / r) * math.sqrt(2.0) / math.sqrt(2.0)
    s1 = (4.0 / r) * math.sqrt(2.0) / math.sqrt(2.0)
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    assert abs(got[0, 0, 0, 0] - p0) <= 1e-14 and abs(got[0, 0, 0, 1] - (1 - p0)) <= 1e-14, got
    rng = _rng(28)
    q = rng.standard_normal((1, 7, 4, 8)); k = rng.standard_normal((1, 7, 2, 8))
    v = rng.standard_normal((1, 7, 2, 8))
    w = (rng.random(8) + 0.5).astype(np.float32)
    a = orc.attention(q, k, v, causal=True, qk_norm=(w, w, 0.0))
    b = orc.attention(q * 37.0, k * 0.01, v, causal=True, qk_norm=(w, w, 0.0))
    assert np.max(np.abs(a - b)) <= 1e-13, np.max(np.abs(a - b))
    assert np.max(np.abs(a - orc.attention(q, k, v, causal=True))) > 1e-3


# ------------------------------------------------------------------------------------------------
# K3 notes, section 4, GVA: H query/key heads shared by HV = G*H value heads
# ------------------------------------------------------------------------------------------------

def check_gva_matches_repeat_interleave_sdpa(orc):
    """Library cross-check of the notes' forward: repeat q and k from H to HV heads with
    torch's repeat_interleave (adjacent copies), then torch fp64 SDPA per value head."""
    import torch
    import torch.nn.functional as F
    rng = _rng(25)
    for (Tq, Tkv, H, HV, causal, W, S) in [(6, 6, 2, 4, True, 0, 0), (5, 5, 1, 3, False, 0, 0),
                                           (4, 9, 3, 6, True, 0, 0), (8, 8, 2, 8, True, 3, 1),
                                           (7, 7, 4, 4, True, 0, 0)]:
        d = 8
        q = rng.standard_normal((2, Tq, H, d)); k = rng.standard_normal((2, Tkv, H, d))
        v = rng.standard_normal((2, Tkv, HV, d))
        got = orc.attention_gva(q, k, v, causal=causal, window=W, n_sink=S)
        G = HV // H
        qt = torch.from_numpy(q).repeat_interleave(G, dim=2).permute(0, 2, 1, 3).contiguous()
        kt = torch.from_numpy(k).repeat_interleave(G, dim=2).permute(0, 2, 1, 3).contiguous()
        vt = torch.from_numpy(v).permute(0, 2, 1, 3).contiguous()
        mask = torch.from_numpy(_window_mask(Tq, Tkv, W if W > 0 else Tkv + 1, S)) if causal \
            else None
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
        err = np.max(np.abs(got - ref.permute(0, 2, 1, 3).numpy()))
        assert err <= 1e-12, (Tq, Tkv, H, HV, causal, W, S, err)


def check_gva_shares_weights_within_a_group(orc):
    """The G value heads of a group use one softmax (the scores of their shared query/key
    head): value heads built as multiples of one base head give the same multiples of its
    output, while the groups differ; G = 1 is multi-head attention, bit for bit."""
    rng = _rng(26)
    H, G, d = 3, 4, 8
    q = rng.standard_normal((1, 7, H, d)); k = rng.standard_normal((1, 7, H, d))
    base = rng.standard_normal((1, 7, H, d))
    v = np.concatenate([base[:, :, h:h + 1] * (m + 1) for h in range(H) for m in range(G)],
                       axis=2)
    out = orc.attention_gva(q, k, v, causal=True)
    for h in range(H):
        for m in range(G):
            err = np.max(np.abs(out[:, :, h * G + m] - (m + 1) * out[:, :, h * G]))
            assert err <= 1e-13 * (m + 1), (h, m, err)
    assert np.max(np.abs(out[:, :, 0] - out[:, :, G])) > 1e-3
    mha = orc.attention(q, k, base, causal=True)
    assert np.array_equal(orc.attention_gva(q, k, base, causal=True), mha)
    # constant values per head: every output row is that constant
    vc = np.broadcast_to(rng.standard_normal((1, 1, H * G, d)), (1, 7, H * G, d)).copy()
    outc = orc.attention_gva(q, k, vc, causal=False)
    assert np.max(np.abs(outc - vc)) <= 1e-14


# ------------------------------------------------------------------------------------------------
# backward (K3 notes, section 4: the gradient of a replicated head is the sum over its copies)
# ------------------------------------------------------------------------------------------------

def check_bwd_matches_torch_autograd(orc):
    """Library cross-check: torch fp64 autograd through repeat_interleave + SDPA (an explicit
    mask table for the causal cases, bottom-right aligned)."""
    import torch
    import torch.nn.functional as F
    rng = _rng(22)
    for (Tq, Tkv, Hq, Hkv, causal, W, S) in [(6, 6, 4, 2, False, 0, 0), (6, 6, 4, 1, True, 0, 0),
                                             (4, 9, 6, 3, True, 0, 0), (7, 7, 2, 2, True, 3, 1),
                                             (5, 5, 8, 2, True, 0, 0)]:
        d = 8
        q = rng.standard_normal((2, Tq, Hq, d)); k = rng.standard_normal((2, Tkv, Hkv, d))
        v = rng.standard_normal((2, Tkv, Hkv, d)); g = rng.standard_normal((2, Tq, Hq, d))
        dq, dk, dv = orc.attention_bwd(q, k, v, g, causal=causal, window=W, n_sink=S)
        G = Hq // Hkv
        qt, kt, vt = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
        mask = torch.from_numpy(_window_mask(Tq, Tkv, W if W > 0 else Tkv + 1, S)) if causal \
            else None
        out = F.scaled_dot_product_attention(
            qt.permute(0, 2, 1, 3), kt.repeat_interleave(G, dim=2).permute(0, 2, 1, 3),
            vt.repeat_interleave(G, dim=2).permute(0, 2, 1, 3), attn_mask=mask)
        (out.permute(0, 2, 1, 3) * torch.from_numpy(g)).sum().backward()
        for name, a, b in (("dq", dq, qt.grad), ("dk", dk, kt.grad), ("dv", dv, vt.grad)):
            err = np.max(np.abs(a - b.numpy()))
            assert err <= 1e-12, (name, Tq, Tkv, Hq, Hkv, causal, W, S, err)


def check_bwd_finite_differences(orc):
    """Central differences of L = sum(out * g) through the (pinned) forward oracle."""
    rng = _rng(23)
    q = rng.standard_normal((1, 4, 4, 4)); k = rng.standard_normal((1, 5, 2, 4))
    v = rng.standard_normal((1, 5, 2, 4)); g = rng.standard_normal((1, 4, 4, 4))
    dq, dk, dv = orc.attention_bwd(q, k, v, g, causal=True)
    h = 1e-6

    def loss(qq, kk, vv):
        return float(np.sum(orc.attention(qq, kk, vv, causal=True) * g))
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for idx in [(0, 0, 0, 0), (0, 3, 1, 2), (0, 2, 0, 3), (0, 1, 1, 1)]:
            if idx[2] >= arr.shape[2] or idx[1] >= arr.shape[1]:
                continue
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += h
            minus[idx] -= h
            args_p = [q, k, v]; args_m = [q, k, v]
            args_p[which] = plus; args_m[which] = minus
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-7, (which, idx, fd, grad[idx])


def check_bwd_invariants(orc):
    """Each row's dS sums to zero over its keys, so the key gradients sum to zero; the value
    gradients sum to the sum of dout (the weights of a row sum to one); constant value rows give
    zero query and key gradients; the G-fold sum rule for key/value heads."""
    rng = _rng(24)
    q = rng.standard_normal((2, 7, 6, 8)); k = rng.standard_normal((2, 7, 2, 8))
    v = rng.standard_normal((2, 7, 2, 8)); g = rng.standard_normal((2, 7, 6, 8))
    dq, dk, dv = orc.attention_bwd(q, k, v, g, causal=True)
    assert np.max(np.abs(dk.sum(axis=1))) <= 1e-12
    gsum = g.reshape(2, 7, 2, 3, 8).sum(axis=(1, 3))          # per key/value head group
    assert np.max(np.abs(dv.sum(axis=1) - gsum)) <= 1e-12
    vc = np.broadcast_to(rng.standard_normal((2, 1, 2, 8)), v.shape).copy()
    dq0, dk0, _ = orc.attention_bwd(q, k, vc, g, causal=True)
    assert np.max(np.abs(dq0)) <= 1e-13 and np.max(np.abs(dk0)) <= 1e-13
    # sum rule: GQA gradients = MHA gradients of the expanded heads, summed over each group
    ke, ve = np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2)
    dqm, dkm, dvm = orc.attention_bwd(q, ke, ve, g, causal=True)
    assert np.max(np.abs(dqm - dq)) <= 1e-12
    assert np.max(np.abs(dkm.reshape(2, 7, 2, 3, 8).sum(axis=3) - dk)) <= 1e-12
    assert np.max(np.abs(dvm.reshape(2, 7, 2, 3, 8).sum(axis=3) - dv)) <= 1e-12


# ------------------------------------------------------------------------------------------------
# lab steps 6-8: exact integer counts (these take the counts module, not the bound oracle)
# ------------------------------------------------------------------------------------------------

def check_counts_lab_scale_exact(counts):
    """Lab step 8's model scale (layers 32, seq_len 4096, head_dim 128, h 8, d_model 1024,
    n_tokens 4096) put through step 6's element count and step 7's per-term multiply count.
    All sizes are powers of two, so the page's formulas reduce to closed forms:
      cache elements 2 * 32 * g * 2^12 * 2^7 = g * 2^25;
      proj_q = proj_out = 2^12 * 2^10 * (8 * 2^7) = 2^32; proj_k = proj_v = g * 2^29;
      scores = weighted = 8 * 2^24 * 2^7 = 2^34; total = 2^30 * (40 + g);
    so kv_ratio = 8 / g and mult_ratio = 48 / (40 + g) (1, 12/11, 8/7, 48/41)."""
    from fractions import Fraction
    table = counts.kv_table(32, 8, [8, 4, 2, 1], 4096, 128)
    assert table == [(8, 268435456), (4, 134217728), (2, 67108864), (1, 33554432)], table
    assert [g * 2 ** 25 for g, _ in table] == [e for _, e in table]
    assert [table[0][1] // e for _, e in table] == [1, 2, 4, 8]
    totals = []
    for g in (8, 4, 2, 1):
        m = counts.mults(4096, 1024, 8, g, 128)
        assert m["proj_q"] == m["proj_out"] == 2 ** 32 == 4294967296, (g, m)
        assert m["proj_k"] == m["proj_v"] == g * 2 ** 29 == 536870912 * g, (g, m)
        assert m["scores"] == m["weighted"] == 2 ** 34 == 17179869184, (g, m)
        assert m["total"] == 2 ** 30 * (40 + g), (g, m)
        assert counts.core_mults(4096, 1024, 8, g, 128) == 2 ** 35
        totals.append(m["total"])
    assert totals == [51539607552, 47244640256, 45097156608, 44023414784]
    assert [Fraction(totals[0], t) for t in totals] == [Fraction(1), Fraction(12, 11),
                                                         Fraction(8, 7), Fraction(48, 41)]


def check_counts_when_heads_times_dim_differs_from_width(counts):
    """Step 7's projection term is tokens x model width x (that projection's heads x head dim);
    at the lab scale h * head_dim equals d_model, so a width-squared projection would go unseen.
    Hand-worked at n = 3, d_model = 5, h = 6, g = 2, head_dim = 7:
      proj_q = proj_out = 3 * 5 * 42 = 630; proj_k = proj_v = 3 * 5 * 14 = 210;
      scores = weighted = 6 * 3 * 3 * 7 = 378; total = 2436.
    And step 6 at layers 3, kv heads 5, length 7, head dim 11: 2 * 3 * 5 * 7 * 11 = 2310."""
    m = counts.mults(3, 5, 6, 2, 7)
    want = {"proj_q": 630, "proj_k": 210, "proj_v": 210, "scores": 378, "weighted": 378,
            "proj_out": 630, "total": 2436}
    assert m == want, m
    assert counts.core_mults(3, 5, 6, 2, 7) == 756
    assert counts.kv_cache_elems(3, 5, 7, 11) == 2310
    assert counts.kv_table(3, 10, [5, 1], 7, 11) == [(5, 2310), (1, 462)]


def check_counts_reject_uneven(counts):
    for bad in (lambda: counts.kv_table(32, 8, [3], 4096, 128),
                lambda: counts.mults(4096, 1024, 8, 3, 128)):
        try:
            bad()
        except ValueError:
            continue
        raise AssertionError("uneven grouping accepted")


COUNT_CHECKS = [
    check_counts_lab_scale_exact,
    check_counts_when_heads_times_dim_differs_from_width,
    check_counts_reject_uneven,
]


ALL_CHECKS = [
    check_group_of_worked_example,
    check_group_of_rejects_uneven,
    check_fold_identity_when_g_is_h,
    check_fold_is_group_mean,
    check_expand_worked_example,
    check_expand_reads_own_group,
    check_matches_torch_sdpa,
    check_scale_is_one_over_sqrt_d,
    check_rows_sum_to_one,
    check_closed_forms,
    check_large_inputs_do_not_overflow,
    check_causality,
    check_window_matches_masked_sdpa,
    check_window_limits,
    check_window_cache_layout,
    check_window_cache_attention,
    check_rope_worked_example,
    check_rope_matches_complex_torch,
    check_rope_relative_positions,
    check_qk_norm_matches_torch_rms_norm,
    check_qk_norm_worked_example_and_scale_invariance,
    check_gva_matches_repeat_interleave_sdpa,
    check_gva_shares_weights_within_a_group,
    check_bwd_matches_torch_autograd,
    check_bwd_finite_differences,
    check_bwd_invariants,
    check_bottom_right_alignment,
    check_g_equals_h_is_mha,
    check_packed_equals_separate,
    check_rows_equal_full,
    check_rows_with_rope_and_norm,
    check_bf16_widening_is_exact,
]
