"""Seeded random shapes against the oracle, through the C ABI: dense, packed and sliding-window
prefill, plain, ragged and windowed decode, decode against caches bounded to the window, grouped
value attention, RoPE and QK-norm (fused or
applied to the keys ahead) and the backward, over head counts, group
sizes, lengths and head dims that the hand-picked cases do not name. The seed fixes the list, so
a failure names a reproducible case (its id carries every size). Inputs are N(0, 1) rounded to
bf16; the bf16 criterion is the one of every other parity test."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_bf16_close, host_view, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

KINDS = ("prefill", "packed", "window", "decode", "ragged", "gva")


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = KINDS[i % len(KINDS)]
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2, 3, 4, 8]))
        g = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 24, 40]))
        while hkv * g > 64:
            g = max(1, g // 2)
        c = {"kind": kind, "d": d, "Hkv": hkv, "G": g, "seed": 7000 + 10 * i}
        if kind == "prefill":
            c["B"] = int(rng.integers(1, 3))
            c["Tkv"] = int(rng.integers(1, 301))
            c["causal"] = bool(rng.integers(0, 2))
            c["Tq"] = int(rng.integers(1, c["Tkv"] + 1)) if rng.integers(0, 2) else c["Tkv"]
        elif kind == "packed":
            lens = [int(x) for x in rng.integers(0, 200, size=int(rng.integers(1, 5)))]
            lens[int(rng.integers(0, len(lens)))] += 1  # at least one token
            c["lens"] = tuple(lens)
            c["causal"] = bool(rng.integers(0, 2))
        elif kind == "window":
            c["T"] = int(rng.integers(1, 301))
            c["window"] = int(rng.integers(1, c["T"] + 20))
            c["n_sink"] = int(rng.integers(0, 9))
        elif kind == "decode":
            c["B"] = int(rng.integers(1, 5))
            c["Tkv"] = int(rng.integers(1, 3001))
        elif kind == "ragged":
            c["B"] = int(rng.integers(2, 6))
            tmax = int(rng.integers(1, 3001))
            c["lens"] = tuple(int(x) for x in rng.integers(1, tmax + 1, size=c["B"]))
            c["Tmax"] = max(c["lens"])
            c["window"] = int(rng.integers(1, tmax + 1)) if rng.integers(0, 2) else 0
            c["n_sink"] = int(rng.integers(0, 9)) if c["window"] else 0
        else:  # gva: H query/key heads, HV = G*H value heads
            c["Hkv"] = int(rng.choice([1, 2, 4]))
            c["G"] = int(rng.choice([1, 2, 3, 4]))
            c["T"] = int(rng.integers(1, 301))
            c["causal"] = bool(rng.integers(0, 2))
        out.append(c)
    return out


CASES = _cases(36, 20261203)


def _id(c):
    return "-".join(f"{k}{v}" for k, v in c.items() if k not in ("seed",)).replace(" ", "")


@pytest.fixture(scope="module")
def gqa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_query_softmax_amd as g
    return g


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("c", CASES, ids=_id)
def test_random_shape_vs_oracle(gqa, orc, c):
    say(f"random shape {_id(c)}")
    d, hkv, s = c["d"], c["Hkv"], c["seed"]
    hq = hkv * c["G"]
    kind = c["kind"]
    if kind == "prefill":
        B, Tq, Tkv = c["B"], c["Tq"], c["Tkv"]
        q = workloads.randn_bf16((B, Tq, hq, d), s)
        k = workloads.randn_bf16((B, Tkv, hkv, d), s + 1)
        v = workloads.randn_bf16((B, Tkv, hkv, d), s + 2)
        got = gqa.gqa_attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=c["causal"])
        ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=c["causal"])
    elif kind == "packed":
        lens = c["lens"]
        tot = sum(lens)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        q = workloads.randn_bf16((1, tot, hq, d), s)
        k = workloads.randn_bf16((1, tot, hkv, d), s + 1)
        v = workloads.randn_bf16((1, tot, hkv, d), s + 2)
        got = gqa.gqa_attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=c["causal"],
                                   cu_seqlens=to_dev(cu), max_seqlen=max(lens))
        ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=c["causal"],
                            cu_seqlens=cu)
    elif kind == "window":
        T, W, S = c["T"], c["window"], c["n_sink"]
        q = workloads.randn_bf16((1, T, hq, d), s)
        k = workloads.randn_bf16((1, T, hkv, d), s + 1)
        v = workloads.randn_bf16((1, T, hkv, d), s + 2)
        got = gqa.gqa_attn_prefill_window(to_dev(q), to_dev(k), to_dev(v), window=W, n_sink=S)
        ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=True, window=W,
                            n_sink=S)
    elif kind == "decode":
        B, Tkv = c["B"], c["Tkv"]
        q = workloads.randn_bf16((B, 1, hq, d), s)
        k = workloads.randn_bf16((B, Tkv, hkv, d), s + 1)
        v = workloads.randn_bf16((B, Tkv, hkv, d), s + 2)
        got = gqa.gqa_attn_decode(to_dev(q), to_dev(k), to_dev(v))
        ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=True)
    elif kind == "ragged":
        B, lens, W, S = c["B"], c["lens"], c["window"], c["n_sink"]
        q = workloads.randn_bf16((B, 1, hq, d), s)
        k = workloads.randn_bf16((B, c["Tmax"], hkv, d), s + 1)
        v = workloads.randn_bf16((B, c["Tmax"], hkv, d), s + 2)
        got = gqa.gqa_attn_decode_ragged(to_dev(q), to_dev(k), to_dev(v),
                                         cache_lens=to_dev(np.asarray(lens, dtype=np.int32)),
                                         window=W, n_sink=S)
        qh, kh, vh = host_view(q), host_view(k), host_view(v)
        ref = np.concatenate([
            orc.attention(qh[b:b + 1], np.ascontiguousarray(kh[b:b + 1, :L]),
                          np.ascontiguousarray(vh[b:b + 1, :L]), causal=True, window=W, n_sink=S)
            for b, L in enumerate(lens)])
    else:
        T, H, HV = c["T"], hkv, hkv * c["G"]
        q = workloads.randn_bf16((1, T, H, d), s)
        k = workloads.randn_bf16((1, T, H, d), s + 1)
        v = workloads.randn_bf16((1, T, HV, d), s + 2)
        got = gqa.gqa_attn_prefill_gva(to_dev(q), to_dev(k), to_dev(v), causal=c["causal"])
        ref = orc.attention_gva(host_view(q), host_view(k), host_view(v), causal=c["causal"])
    torch.cuda.synchronize()
    assert_bf16_close(to_f64(got), ref, what=_id(c))


def _wc_cases(n, seed):
    """Decode against caches bounded to the window: window, sinks and entry counts drawn so that
    some caches are empty, some not yet full, some written over many times."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2, 3, 4, 8]))
        g = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 24, 40]))
        while hkv * g > 64:
            g = max(1, g // 2)
        B = int(rng.integers(1, 6))
        W = int(rng.integers(1, 1500))
        S = int(rng.integers(0, 9)) if rng.integers(0, 3) else int(rng.integers(0, 200))
        lens = tuple(int(x) for x in rng.integers(0, 4 * (W + S) + 2, size=B))
        out.append({"d": d, "Hkv": hkv, "G": g, "B": B, "window": W, "n_sink": S, "lens": lens,
                    "seed": 9100 + 10 * i})
    return out


WC_CASES = _wc_cases(12, 20261206)


def _wc_id(c):
    return "wc_B{B}_W{window}_S{n_sink}_Hkv{Hkv}_G{G}_d{d}_s{seed}".format(**c)


@pytest.mark.parametrize("c", WC_CASES, ids=_wc_id)
def test_random_window_cache_vs_oracle(gqa, orc, c):
    B, W, S, d, seed = c["B"], c["window"], c["n_sink"], c["d"], c["seed"]
    hkv, hq = c["Hkv"], c["Hkv"] * c["G"]
    say(_wc_id(c))
    q = workloads.randn_bf16((B, 1, hq, d), seed)
    k = workloads.randn_bf16((B, S + W, hkv, d), seed + 1)
    v = workloads.randn_bf16((B, S + W, hkv, d), seed + 2)
    lens = np.asarray(c["lens"], dtype=np.int32)
    got = to_f64(gqa.gqa_attn_decode_window_cache(to_dev(q), to_dev(k), to_dev(v), to_dev(lens),
                                                  window=W, n_sink=S))
    torch.cuda.synchronize()
    qh = host_view(q)
    kc = oracle.unroll_window_cache(host_view(k), c["lens"], W, S, compact=True)
    vc = oracle.unroll_window_cache(host_view(v), c["lens"], W, S, compact=True)
    for b, L in enumerate(c["lens"]):
        if L == 0:
            assert np.array_equal(got[b], np.zeros_like(got[b])), f"{_wc_id(c)} seq {b}: empty"
            continue
        ref = orc.attention(qh[b:b + 1], kc[b], vc[b])
        assert_bf16_close(got[b:b + 1], ref, what=f"{_wc_id(c)} seq {b} len {L}")


def _bwd_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 3, 4, 6, 8]))
        tkv = int(rng.integers(1, 257))
        causal = bool(rng.integers(0, 2))
        tq = int(rng.integers(1, tkv + 1)) if rng.integers(0, 2) else tkv
        out.append({"B": int(rng.integers(1, 3)), "Tq": tq, "Tkv": tkv, "Hkv": hkv, "G": g,
                    "d": int(rng.choice([64, 128])), "causal": causal, "seed": 7500 + 10 * i})
    return out


BWD_CASES = _bwd_cases(12, 20261204)
GRAD_REL = 1e-2  # rel-to-max per gradient, as for the hand-picked backward cases


@pytest.mark.parametrize("c", BWD_CASES, ids=_id)
def test_random_backward_vs_oracle(gqa, orc, c):
    """dq, dk, dv of sum(out * dout) for random dense shapes; the GPU backward reads the GPU
    forward's output and row log-sum-exp, as a training step does."""
    say(f"random backward {_id(c)}")
    B, Tq, Tkv, hkv, d, s = c["B"], c["Tq"], c["Tkv"], c["Hkv"], c["d"], c["seed"]
    hq = hkv * c["G"]
    q = workloads.randn_bf16((B, Tq, hq, d), s)
    k = workloads.randn_bf16((B, Tkv, hkv, d), s + 1)
    v = workloads.randn_bf16((B, Tkv, hkv, d), s + 2)
    g = workloads.randn_bf16((B, Tq, hq, d), s + 3)
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    lse = torch.empty(B, Tq, hq, dtype=torch.float32, device="cuda")
    out = gqa.gqa_attn_prefill_ex(qd, kd, vd, causal=c["causal"], lse=lse)
    dq, dk, dv = gqa.gqa_attn_backward(qd, kd, vd, out, gd, lse, causal=c["causal"])
    torch.cuda.synchronize()
    refs = orc.attention_bwd(host_view(q), host_view(k), host_view(v), host_view(g),
                             causal=c["causal"])
    # Each gradient's error is taken relative to its own largest value. Only where the exact
    # gradient is zero everywhere (every row sees a single key, so P = 1 and dS = P (dP - D)
    # vanishes, making dq and dk exactly 0) is there no own scale: there the GPU's rounding noise
    # is measured against dv's largest value (the weighted dout, the gradients' natural scale).
    scale_dv = float(np.max(np.abs(refs[2])))
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        got = to_f64(got)
        assert np.all(np.isfinite(got)), name
        own = float(np.max(np.abs(ref)))
        denom = own if own > 0 else scale_dv
        err = float(np.max(np.abs(got - ref)) / denom)
        assert err <= GRAD_REL, f"{_id(c)} {name}: rel-to-max {err:.3g} (own max {own:.3g})"


def _proc_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = ("fused", "prepared", "decode")[i % 3]
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 3, 4, 8]))
        rope = bool(rng.integers(0, 2))
        norm = bool(rng.integers(0, 2)) or not rope  # at least one of the two
        c = {"kind": kind, "d": int(rng.choice([64, 128])), "Hkv": hkv, "G": g, "rope": rope,
             "norm": norm, "seed": 7800 + 10 * i}
        if kind == "decode":
            c["B"] = int(rng.integers(1, 4))
            c["Tkv"] = int(rng.integers(1, 2001))
        else:
            c["B"] = int(rng.integers(1, 3))
            c["Tkv"] = int(rng.integers(1, 301))
            c["Tq"] = int(rng.integers(1, c["Tkv"] + 1)) if rng.integers(0, 2) else c["Tkv"]
            c["causal"] = bool(rng.integers(0, 2)) if kind == "fused" else True
        out.append(c)
    return out


PROC_CASES = _proc_cases(12, 20261205)
EPS = 1e-6


@pytest.mark.parametrize("c", PROC_CASES, ids=_id)
def test_random_rope_qknorm_vs_oracle(gqa, orc, c):
    """RoPE and/or QK-norm: fused into prefill, applied to the keys once by gqa_prepare_keys
    before a keys_prepared prefill, or applied to a decode cache before decode. The oracle
    processes the raw q and k itself in every case."""
    say(f"random rope/qk-norm {_id(c)}")
    d, hkv, s, kind = c["d"], c["Hkv"], c["seed"], c["kind"]
    hq, B, Tkv = hkv * c["G"], c["B"], c["Tkv"]
    Tq = 1 if kind == "decode" else c["Tq"]
    rng = np.random.default_rng(s + 3)
    wq = (rng.random(d) * 1.5 + 0.25).astype(np.float32)
    wk = (rng.random(d) * 1.5 + 0.25).astype(np.float32)
    tabs = workloads.rope_tables(Tkv, d) if c["rope"] else None
    dt = tuple(to_dev(t) for t in tabs) if c["rope"] else None
    q = workloads.randn_bf16((B, Tq, hq, d), s)
    k = workloads.randn_bf16((B, Tkv, hkv, d), s + 1)
    v = workloads.randn_bf16((B, Tkv, hkv, d), s + 2)
    dwq, dwk = to_dev(wq), to_dev(wk)
    norm = c["norm"]
    causal = c.get("causal", True)
    if kind == "fused":
        got = gqa.gqa_attn_prefill_ex(to_dev(q), to_dev(k), to_dev(v), causal=causal, rope=dt,
                                      qk_norm=(dwq, dwk, EPS) if norm else None)
    elif kind == "prepared":
        kp = gqa.gqa_prepare_keys(to_dev(k), rope=dt, qk_norm=(None, dwk, EPS) if norm else None)
        got = gqa.gqa_attn_prefill_ex(to_dev(q), kp, to_dev(v), causal=True, rope=dt,
                                      qk_norm=(dwq, None, EPS) if norm else None,
                                      keys_prepared=True)
    else:
        kc = gqa.gqa_prepare_keys(to_dev(k), rope=dt, qk_norm=(None, dwk, EPS) if norm else None)
        lens = np.full(B, Tkv, dtype=np.int32)
        got = gqa.gqa_attn_decode_ex(to_dev(q), kc, to_dev(v), cache_lens=to_dev(lens), rope=dt,
                                     qk_norm=(dwq, None, EPS) if norm else None)
    torch.cuda.synchronize()
    ref = orc.attention(host_view(q), host_view(k), host_view(v), causal=causal, rope=tabs,
                        qk_norm=(wq, wk, EPS) if norm else None)
    assert_bf16_close(to_f64(got), ref, what=_id(c))
