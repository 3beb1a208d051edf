"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The benchmark workloads (the 4096-token 32/8 prefill, the 64-sequence decode, the multi-query
prefill with its x30 rows, the packed 16k/8k/4k/1k prefill, the long-context decode of one
131072-entry cache, which runs split and merges its partial results, and the decode against caches
bounded to the window) are compared with the fp64
oracle over the whole output, every head, row and column (the GQA lab's max_gap, step 5; the course
page's whole-output comparison with torch's scaled_dot_product_attention). The variant workloads
(window, ragged decode, rotary embedding, grouped values, backward) are checked on seeded
samples of rows, sequences or head groups; rows are independent, so each sampled row is an exact
check of that row."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_bf16_close, host_view, say, to_dev, to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def gqa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_query_softmax_amd as g
    return g


def _whole(got, ref, what):
    err, rel = assert_bf16_close(got, ref, what=what)
    say(f"{what}: whole output max-abs {err:.3e} rel-to-max {rel:.3e}")
    return err, rel


def _dense_prefill(gqa, w):
    q, k, v, _ = workloads.make_inputs(w)
    say(f"full-size prefill {w.name}: launching")
    out = gqa.gqa_attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=w.causal)
    torch.cuda.synchronize()
    return q, k, v, to_f64(out)


def test_full_llama_prefill_whole_output(gqa):
    """The 4096-token 32/8 causal prefill: every head, row and column against the fp64 oracle
    (the GQA lab's max_gap over the whole output, step 5)."""
    w = workloads.LLAMA_PREFILL
    q, k, v, got = _dense_prefill(gqa, w)
    say(f"full-size prefill {w.name}: oracle on the whole output")
    ref = oracle.default().attention(host_view(q), host_view(k), host_view(v), causal=True)
    _whole(got, ref, w.name)


def test_full_mqa_prefill_whole_output(gqa):
    """The 8 x 2048-token multi-query prefill with 5 % of the query rows scaled x30: the whole
    output, and separately every scaled (peaked) row."""
    w = workloads.MQA_PREFILL
    q, k, v, got = _dense_prefill(gqa, w)
    say(f"full-size prefill {w.name}: oracle on the whole output")
    ref = oracle.default().attention(host_view(q), host_view(k), host_view(v), causal=True)
    _whole(got, ref, w.name)
    pk = workloads.peaked_rows(w)
    assert len(pk) == 26214
    g2 = got.reshape(-1, w.d)[pk]
    r2 = ref.reshape(-1, w.d)[pk]
    _whole(g2, r2, f"{w.name} (the {len(pk)} x30 rows)")


def test_full_decode_whole_output(gqa):
    """The 64-sequence decode against 8192-entry caches: every sequence, head and column (the
    oracle runs a few sequences at a time to bound its expanded key/value copies)."""
    w = workloads.DECODE
    say("full-size decode: generating inputs")
    q, k, v, _ = workloads.make_inputs(w)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    ws = torch.empty(gqa.gqa_attn_decode_workspace_bytes(w.B, w.Tkv, w.Hq, w.d),
                     dtype=torch.uint8, device="cuda")
    say("full-size decode: launching")
    out = gqa.gqa_attn_decode(qd, kd, vd, workspace=ws)
    torch.cuda.synchronize()
    got = to_f64(out)
    qh, kh, vh = host_view(q), host_view(k), host_view(v)
    orc = oracle.default()
    ref = np.empty_like(got)
    step = 8
    for b0 in range(0, w.B, step):
        say(f"full-size decode: oracle on sequences {b0} .. {b0 + step - 1}")
        ref[b0:b0 + step] = orc.attention(qh[b0:b0 + step], kh[b0:b0 + step], vh[b0:b0 + step])
    _whole(got, ref, w.name)


def test_full_long_decode_whole_output(gqa):
    """One sequence against a 131072-entry cache: the cache is split across the compute units and
    the partial results are merged by the combine kernel; every head and column is compared."""
    w = workloads.LONG_DECODE
    splits = (gqa.raw_library().gqa_attn_decode_workspace_bytes_hkv(w.B, w.Tkv, w.Hq, w.Hkv, w.d)
              // (w.B * w.Hq * (w.d + 2) * 4))
    assert splits > 1, "the long-context decode must run split (and merge the partials)"
    say(f"full-size long decode {w.name}: generating inputs")
    q, k, v, _ = workloads.make_inputs(w)
    ws = torch.empty(gqa.gqa_attn_decode_workspace_bytes(w.B, w.Tkv, w.Hq, w.d),
                     dtype=torch.uint8, device="cuda")
    say(f"full-size long decode: launching ({splits} splits)")
    out = gqa.gqa_attn_decode(to_dev(q), to_dev(k), to_dev(v), workspace=ws)
    torch.cuda.synchronize()
    got = to_f64(out)
    say("full-size long decode: oracle on the whole output")
    ref = oracle.default().attention(host_view(q), host_view(k), host_view(v))
    _whole(got, ref, w.name)


def test_full_window_cache_decode_whole_output(gqa):
    """64 sequences of 32768 entries each in caches bounded to a 4096-entry window and 4 sinks
    (4100 slots, written over about eight times): every sequence, head and column against the
    oracle, which reads each visible entry back from its slot (course page "Week 7. Attention",
    step 3)."""
    w = workloads.WINDOW_CACHE_DECODE
    say(f"full-size window-cache decode {w.name}: generating inputs")
    q, k, v, _ = workloads.make_inputs(w)
    lens = torch.tensor(w.cache_lens, dtype=torch.int32, device="cuda")
    say("full-size window-cache decode: launching")
    out = gqa.gqa_attn_decode_window_cache(to_dev(q), to_dev(k), to_dev(v), lens,
                                           window=w.window, n_sink=w.n_sink)
    torch.cuda.synchronize()
    got = to_f64(out)
    qh = host_view(q)
    kc = oracle.unroll_window_cache(host_view(k), w.cache_lens, w.window, w.n_sink, compact=True)
    vc = oracle.unroll_window_cache(host_view(v), w.cache_lens, w.window, w.n_sink, compact=True)
    say("full-size window-cache decode: oracle on every sequence")
    orc = oracle.default()
    ref = np.concatenate([orc.attention(qh[b:b + 1], kc[b], vc[b]) for b in range(w.B)])
    _whole(got, ref, w.name)


# The packed 16k/8k/4k/1k prefill is checked whole, in slices of one sequence and a block of
# key/value heads (with their query heads), so that each test's oracle run stays under a minute.
VARLEN_SLICES = [(0, j, j + 1) for j in range(8)] + [(1, 0, 4), (1, 4, 8), (2, 0, 8), (3, 0, 8)]


@pytest.fixture(scope="module")
def varlen_run(gqa):
    w = workloads.VARLEN_PREFILL
    say(f"full-size prefill {w.name}: generating inputs")
    q, k, v, cu = workloads.make_inputs(w)
    say(f"full-size prefill {w.name}: launching")
    out = gqa.gqa_attn_prefill(to_dev(q), to_dev(k), to_dev(v), causal=True,
                               cu_seqlens=to_dev(cu), max_seqlen=max(w.seqlens))
    torch.cuda.synchronize()
    return w, host_view(q), host_view(k), host_view(v), cu, out.cpu()


@pytest.mark.slow
@pytest.mark.parametrize("sl", VARLEN_SLICES, ids=lambda s: f"seq{s[0]}_kv{s[1]}-{s[2] - 1}")
def test_full_varlen_prefill_whole_output(varlen_run, sl):
    w, qh, kh, vh, cu, out = varlen_run
    s, j0, j1 = sl
    G = w.Hq // w.Hkv
    a, b = int(cu[s]), int(cu[s + 1])
    hs = slice(j0 * G, j1 * G)
    say(f"full-size prefill {w.name}: oracle on sequence {s}, key/value heads {j0} .. {j1 - 1}")
    ref = oracle.default().attention(np.ascontiguousarray(qh[:, a:b, hs]),
                                     np.ascontiguousarray(kh[:, a:b, j0:j1]),
                                     np.ascontiguousarray(vh[:, a:b, j0:j1]), causal=True)
    _whole(to_f64(out[:, a:b, hs]), ref, f"{w.name} seq {s} kv {j0}-{j1 - 1}")


def test_full_window_prefill_sampled_rows(gqa):
    w = workloads.WINDOW_PREFILL
    say(f"full-size window prefill {w.name}: generating inputs")
    q, k, v, _ = workloads.make_inputs(w)
    say(f"full-size window prefill {w.name}: launching")
    out = gqa.gqa_attn_prefill_window(to_dev(q), to_dev(k), to_dev(v), window=w.window,
                                      n_sink=w.n_sink)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    rows = workloads.sample_rows(w, 160, seed=10)
    say(f"full-size window prefill: oracle on {len(rows)} rows")
    ref = oracle.default().attention_rows(host_view(q), host_view(k), host_view(v), rows,
                                          causal=True, window=w.window, n_sink=w.n_sink)
    o = out.cpu()
    got = np.stack([to_f64(o[b, t, h]) for b, t, h in rows])
    err, rel = assert_bf16_close(got, ref, what=w.name)
    say(f"full-size window prefill: max-abs {err:.3e} rel {rel:.3e}")


def test_full_ragged_decode_sampled_sequences(gqa):
    w = workloads.RAGGED_DECODE
    say(f"full-size ragged decode {w.name}: generating inputs")
    q, k, v, _ = workloads.make_inputs(w)
    lens = torch.tensor(w.cache_lens, dtype=torch.int32).cuda()
    ws = torch.empty(gqa.gqa_attn_decode_workspace_bytes(w.B, w.Tkv, w.Hq, w.d),
                     dtype=torch.uint8, device="cuda")
    say("full-size ragged decode: launching")
    out = gqa.gqa_attn_decode_ragged(to_dev(q), to_dev(k), to_dev(v), cache_lens=lens,
                                     workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    got = to_f64(out)
    qh, kh, vh = host_view(q), host_view(k), host_view(v)
    # the shortest and longest sequences plus a seeded sample of the rest, all heads
    pick = sorted({0, w.B - 1, *np.random.default_rng(11).choice(w.B, 6, replace=False).tolist()})
    say(f"full-size ragged decode: oracle on sequences {pick}")
    orc = oracle.default()
    for b in pick:
        L = w.cache_lens[b]
        ref = orc.attention(qh[b:b + 1], np.ascontiguousarray(kh[b:b + 1, :L]),
                            np.ascontiguousarray(vh[b:b + 1, :L]), causal=True)
        assert_bf16_close(got[b:b + 1], ref, what=f"{w.name} seq {b} len {L}")


def test_full_rope_prefill_sampled_rows(gqa):
    """The headline prefill with the rotary embedding fused into the kernel."""
    w = workloads.LLAMA_PREFILL
    say("full-size rope prefill: generating inputs")
    q, k, v, _ = workloads.make_inputs(w)
    cos_t, sin_t = workloads.rope_tables(w.Tkv, w.d)
    say("full-size rope prefill: launching")
    out = gqa.gqa_attn_prefill_ex(to_dev(q), to_dev(k), to_dev(v), causal=True,
                                  rope=(to_dev(cos_t), to_dev(sin_t)))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    rows = workloads.sample_rows(w, 160, seed=12)
    say(f"full-size rope prefill: oracle on {len(rows)} rows")
    ref = oracle.default().attention_rows(host_view(q), host_view(k), host_view(v), rows,
                                          causal=True, rope=(cos_t, sin_t))
    o = out.cpu()
    got = np.stack([to_f64(o[b, t, h]) for b, t, h in rows])
    err, rel = assert_bf16_close(got, ref, what="rope prefill")
    say(f"full-size rope prefill: max-abs {err:.3e} rel {rel:.3e}")


def test_full_gva_prefill_sampled_heads(gqa):
    """Grouped value attention at the benchmark size: the first and last query/key head of every
    sequence, with all of their value heads and every position, against the fp64 oracle."""
    w = workloads.GVA_PREFILL
    H, HV = w.Hkv, w.Hq
    G = HV // H
    say(f"full-size gva {w.name}: generating inputs")
    q, k, v = workloads.gva_inputs(w)
    say(f"full-size gva {w.name}: launching")
    out = gqa.gqa_attn_prefill_gva(to_dev(q), to_dev(k), to_dev(v), causal=w.causal)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    o = out.cpu()
    orc = oracle.default()
    qh, kh, vh = host_view(q), host_view(k), host_view(v)
    for b in range(w.B):
        for h in (0, H - 1):
            say(f"full-size gva {w.name}: oracle on sequence {b}, query/key head {h}")
            ref = orc.attention_gva(qh[b:b + 1, :, h:h + 1], kh[b:b + 1, :, h:h + 1],
                                    vh[b:b + 1, :, h * G:(h + 1) * G], causal=w.causal)
            assert_bf16_close(to_f64(o[b:b + 1, :, h * G:(h + 1) * G]), ref,
                              what=f"{w.name} b={b} h={h}")


def test_full_backward_sampled_groups(gqa):
    """Backward at the benchmark size (T = 4096, 32/8, causal): the gradients of the first and
    last key/value-head group (its 4 query heads, every position) against the fp64 oracle run
    on that group alone (a group's dq, dk, dv depend only on its own heads)."""
    w = workloads.LLAMA_PREFILL
    G = w.Hq // w.Hkv
    say("full-size backward: generating inputs")
    q, k, v, _ = workloads.make_inputs(w)
    g = workloads.randn_bf16((w.B, w.Tq, w.Hq, w.d), 2099)
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    lse = torch.empty(w.B, w.Tq, w.Hq, dtype=torch.float32, device="cuda")
    say("full-size backward: forward + backward")
    out = gqa.gqa_attn_prefill_ex(qd, kd, vd, causal=True, lse=lse)
    dq, dk, dv = gqa.gqa_attn_backward(qd, kd, vd, out, gd, lse, causal=True)
    torch.cuda.synchronize()
    orc = oracle.default()
    qh, kh, vh, gh = host_view(q), host_view(k), host_view(v), host_view(g)
    for j in (0, w.Hkv - 1):
        say(f"full-size backward: oracle on key/value head {j}")
        hs = slice(j * G, (j + 1) * G)
        rq, rk, rv = orc.attention_bwd(qh[:, :, hs], kh[:, :, j:j + 1], vh[:, :, j:j + 1],
                                       gh[:, :, hs], causal=True)
        for name, got, ref in (("dq", dq[:, :, hs], rq), ("dk", dk[:, :, j:j + 1], rk),
                               ("dv", dv[:, :, j:j + 1], rv)):
            e = float(np.max(np.abs(to_f64(got) - ref)) / np.max(np.abs(ref)))
            say(f"full-size backward head {j} {name}: rel-to-max {e:.3e}")
            assert np.all(np.isfinite(to_f64(got))) and e <= 1e-2, (j, name, e)
