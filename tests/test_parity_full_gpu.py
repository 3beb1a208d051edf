"""GPU parity at the full workload sizes, in the launch configuration the benchmark times:
the whole output is computed on the GPU, and a seeded sample of output rows (always including
the first and last position of every batch item / packed sequence, for the first and last head,
plus -- for the MQA workload -- a sample of the x30 rows) is recomputed one by one by the fp64
oracle. Rows are independent, so each sampled row is an exact check of that row."""
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


def _check_rows(w, q, k, v, cu, out, rows):
    orc = oracle.default()
    ref = orc.attention_rows(host_view(q), host_view(k), host_view(v), rows, causal=w.causal,
                             cu_seqlens=cu)
    o = out.cpu()
    got = np.stack([to_f64(o[b, t, h]) for b, t, h in rows])
    return assert_bf16_close(got, ref, what=w.name)


@pytest.mark.parametrize("w", [workloads.LLAMA_PREFILL, workloads.MQA_PREFILL,
                               workloads.VARLEN_PREFILL], ids=lambda w: w.name)
def test_full_prefill_sampled_rows(gqa, w):
    say(f"full-size prefill {w.name}: generating inputs")
    q, k, v, cu = workloads.make_inputs(w)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    cud = to_dev(cu) if cu is not None else None
    say(f"full-size prefill {w.name}: launching")
    out = gqa.gqa_attn_prefill(qd, kd, vd, causal=w.causal, cu_seqlens=cud,
                               max_seqlen=max(w.seqlens) if w.seqlens else None)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    rows = workloads.sample_rows(w, 160, seed=7)
    if w.peaked_frac > 0:
        pk = workloads.peaked_rows(w)
        sel = np.random.default_rng(8).choice(pk, size=96, replace=False)
        extra = np.stack([sel // (w.Tq * w.Hq), (sel // w.Hq) % w.Tq, sel % w.Hq], axis=1)
        rows = np.unique(np.concatenate([rows, extra]), axis=0)
    say(f"full-size prefill {w.name}: oracle on {len(rows)} rows")
    err, rel = _check_rows(w, q, k, v, cu, out, rows)
    say(f"full-size prefill {w.name}: max-abs {err:.3e} rel {rel:.3e}")


def test_full_decode_sampled_rows(gqa):
    w = workloads.DECODE
    say("full-size decode: generating inputs")
    q, k, v, _ = workloads.make_inputs(w)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    ws = torch.empty(gqa.gqa_attn_decode_workspace_bytes(w.B, w.Tkv, w.Hq, w.Hkv, w.d),
                     dtype=torch.uint8, device="cuda")
    say("full-size decode: launching")
    out = gqa.gqa_attn_decode(qd, kd, vd, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    rows = workloads.sample_rows(w, 200, seed=9)
    say(f"full-size decode: oracle on {len(rows)} rows")
    err, rel = _check_rows(w, q, k, v, None, out, rows)
    say(f"full-size decode: max-abs {err:.3e} rel {rel:.3e}")


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
    ws = torch.empty(gqa.gqa_attn_decode_workspace_bytes(w.B, w.Tkv, w.Hq, w.Hkv, w.d),
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
