"""GPU (HIP, through the C ABI) against the float64 oracle on identical inputs.

Small cases compare every element; the full-size workloads compare the
outputs the oracle can compute at that size (whole KV groups, sampled rows
and keys) and check the rest through identities that hold at any size.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synthetic.workloads import WORKLOADS, custom_workload, make_inputs, make_inputs_device
from tests.parity_util import (TOL_DS, TOL_GRAD, TOL_LSE, TOL_O, check_full, f64, max_abs,
                               record_errors, rel_l2, run_gpu, say)

pytestmark = pytest.mark.gpu


def _oracle_full(inp, scale, window):
    q, k, v, do, s, cu = (inp[n] for n in ("q", "k", "v", "dout", "sinks", "cu_seqlens"))
    o, lse = oracle.forward(q, k, v, s, cu, scale, window)
    dq, dk, dv, ds = oracle.backward(q, k, v, s, do, cu, scale, window)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "ds": ds}


def _set_sinks(inp, mode, hq):
    if mode == "minus_inf":
        inp["sinks"] = torch.full((hq,), -math.inf)
    elif mode == "plus30":
        inp["sinks"] = torch.full((hq,), 30.0)
    elif mode == "mixed":
        vals = [-math.inf, 0.0, 5.0, 30.0, -3.0, 1.5, -math.inf, 2.0]
        inp["sinks"] = torch.tensor([vals[i % len(vals)] for i in range(hq)], dtype=torch.float32)
    return inp


SMALL = [
    # lengths, hq, hkv, d, window, dtype, sinks
    ((1,), 4, 2, 64, 0, "bf16", "normal"),
    ((2,), 4, 2, 64, 0, "bf16", "normal"),
    ((63,), 8, 1, 64, 0, "bf16", "normal"),
    ((65,), 8, 8, 64, 0, "bf16", "normal"),
    ((127,), 4, 2, 32, 0, "bf16", "normal"),
    ((129,), 4, 1, 64, 0, "bf16", "normal"),
    ((300,), 8, 2, 64, 0, "bf16", "normal"),
    ((0, 5, 1, 130, 0, 64, 257), 4, 2, 64, 0, "bf16", "normal"),
    ((200,), 4, 2, 64, 1, "bf16", "normal"),
    ((300,), 4, 2, 64, 17, "bf16", "normal"),
    ((333, 129), 8, 1, 64, 128, "bf16", "normal"),
    ((150,), 2, 1, 64, 1000, "bf16", "normal"),
    ((129, 70), 4, 2, 16, 0, "bf16", "normal"),
    ((100,), 4, 2, 64, 0, "bf16", "minus_inf"),
    ((100,), 4, 2, 64, 0, "bf16", "plus30"),
    ((190,), 8, 2, 64, 0, "bf16", "mixed"),
    ((257,), 4, 2, 40, 0, "f32", "normal"),
    ((200, 3), 4, 4, 64, 9, "f32", "mixed"),
    ((520,), 16, 2, 64, 0, "bf16", "normal"),
    # windows of at most 128 keys run the forward on 32-key tiles, longer
    # ones on 64-key tiles: both sides of that boundary and of one tile
    ((301,), 8, 1, 64, 31, "bf16", "normal"),
    ((301,), 8, 1, 64, 32, "bf16", "mixed"),
    ((301,), 8, 1, 64, 33, "bf16", "normal"),
    ((260, 77), 16, 2, 64, 127, "bf16", "normal"),
    ((260,), 16, 2, 64, 129, "bf16", "normal"),
    ((190,), 4, 2, 40, 128, "f32", "normal"),
    ((190,), 4, 2, 32, 64, "bf16", "minus_inf"),
    # groups that are not a power of two (3 and 6 query heads per KV head)
    ((260, 33), 6, 2, 64, 0, "bf16", "normal"),
    ((300,), 12, 2, 64, 50, "bf16", "mixed"),
    ((97, 131), 6, 1, 32, 0, "f32", "normal"),
    ((129,), 1, 1, 64, 0, "bf16", "normal"),
]


@pytest.mark.parametrize("lengths,hq,hkv,d,window,dtype,sinks", SMALL)
def test_small_cases_match_oracle(lengths, hq, hkv, d, window, dtype, sinks):
    label = f"L={lengths} hq={hq} hkv={hkv} d={d} W={window} {dtype} sinks={sinks}"
    say("case", label)
    w = custom_workload(lengths, hq, hkv, d, window, dtype)
    inp = _set_sinks(make_inputs(w, seed=sum(lengths) + 7 * hq + d), sinks, hq)
    scale = 1.0 / math.sqrt(d)
    gpu = run_gpu(inp, w.max_seqlen, scale, window)
    ref = _oracle_full(inp, scale, window)
    check_full(gpu, ref, label)
    if sinks == "minus_inf":
        assert np.all(gpu["ds"] == 0.0)


GROUPED = [
    # lengths, hq, hkv, d, window, dtype, sinks: dK/dV workgroups covering
    # every query head of a KV group (direct dK, dV stores) and some of them
    ((1,), 4, 2, 64, 0, "bf16", "normal"),
    ((300,), 8, 2, 64, 0, "bf16", "mixed"),
    ((0, 5, 1, 130, 0, 64, 257), 4, 2, 64, 0, "bf16", "normal"),
    ((333, 129), 8, 1, 64, 128, "bf16", "normal"),
    ((129, 70), 4, 2, 16, 0, "bf16", "normal"),
    ((200, 3), 4, 2, 40, 9, "f32", "mixed"),
    ((520,), 16, 2, 64, 0, "bf16", "normal"),
    # windows of at most 128 keys run the forward on 32-key tiles, longer
    # ones on 64-key tiles: both sides of that boundary and of one tile
    ((301,), 8, 1, 64, 31, "bf16", "normal"),
    ((301,), 8, 1, 64, 32, "bf16", "mixed"),
    ((301,), 8, 1, 64, 33, "bf16", "normal"),
    ((260, 77), 16, 2, 64, 127, "bf16", "normal"),
    ((260,), 16, 2, 64, 129, "bf16", "normal"),
    ((190,), 4, 2, 40, 128, "f32", "normal"),
    ((190,), 4, 2, 32, 64, "bf16", "minus_inf"),
]


@pytest.mark.parametrize("heads", ["group", 2])
@pytest.mark.parametrize("lengths,hq,hkv,d,window,dtype,sinks", GROUPED)
def test_grouped_dkdv_workgroups_match_oracle(monkeypatch, heads, lengths, hq, hkv, d, window, dtype, sinks):
    hg = hq // hkv if heads == "group" else heads
    if (hq // hkv) % hg:
        pytest.skip("head count does not divide the group")
    monkeypatch.setenv("SINK_ATTN_DKDV_HEADS", str(hg))
    label = f"L={lengths} hq={hq} hkv={hkv} d={d} W={window} {dtype} sinks={sinks} dkdv_heads={hg}"
    say("case", label)
    w = custom_workload(lengths, hq, hkv, d, window, dtype)
    inp = _set_sinks(make_inputs(w, seed=sum(lengths) + 7 * hq + d + 1), sinks, hq)
    scale = 1.0 / math.sqrt(d)
    gpu = run_gpu(inp, w.max_seqlen, scale, window)
    ref = _oracle_full(inp, scale, window)
    check_full(gpu, ref, label)


def large_logit_inputs(factor, window, seed=77):
    """Keys 100..119 and 250..259 (packed rows) scaled by `factor`: the scores
    of later rows jump far above the running maximum.  softmax_scale is
    0.125 / log2(e), so the forward's scaled query operand (q * scale *
    log2 e = q / 8) is exact in bf16 and the large scores carry no rounding
    beyond the float accumulation."""
    w = custom_workload((300, 130), 8, 2, 64, window, "bf16")
    inp = make_inputs(w, seed=seed + int(factor) + window)
    k = inp["k"].float()
    k[100:120] *= factor
    k[250:260] *= factor
    inp["k"] = k.to(inp["k"].dtype)
    return w, inp, 0.125 / math.log2(math.e)


@pytest.mark.parametrize("factor", [8.0, 80.0])
@pytest.mark.parametrize("window", [0, 40])
def test_large_logit_jumps_match_oracle(factor, window):
    """Score jumps of about 20 (factor 8) and over 128 (factor 80) log2 units
    above a row's running maximum: the forward raises its reference by an
    integer power of two, or (an overflowing tile) by the exact tile maximum."""
    w, inp, scale = large_logit_inputs(factor, window)
    label = f"large logits x{factor} W={window}"
    say("case", label)
    gpu = run_gpu(inp, w.max_seqlen, scale, window)
    check_full(gpu, _oracle_full(inp, scale, window), label)


def very_negative_first_tile_inputs(window, seed=91):
    """Sink -inf, queries near (1, ..., 1), the first 64 keys of each
    sequence equal to -0.6 * (1, ..., 1) and softmax_scale = 4 / log2(e):
    every row's first key tile scores between about -175 and -135 log2 units
    (q . k * scale * log2 e = 4 q . k, exact in the bf16 scaled query), far
    below -128.  A row's reference is -inf until that tile, so the forward's
    first rescale must not form exp2(+150) = inf.  The later keys are
    0.1 * N(0, 1), so their scores spread over a few log2 units only (keys of
    ordinary size: a large common key offset would amplify the bf16 rounding
    of dS into dQ rows whose exact value cancels)."""
    w = custom_workload((300, 130), 8, 2, 64, window, "bf16")
    inp = make_inputs(w, seed=seed + window)
    inp["q"] = (1.0 + 0.25 * inp["q"].float()).to(torch.bfloat16)
    k = 0.1 * inp["k"].float()
    for b in (0, 300):
        k[b:b + 64] = -0.6
    inp["k"] = k.to(torch.bfloat16)
    inp["sinks"] = torch.full((8,), -math.inf)
    return w, inp, 4.0 / math.log2(math.e)


@pytest.mark.parametrize("window", [0, 40])
def test_minus_inf_sink_with_very_negative_first_tile(window):
    w, inp, scale = very_negative_first_tile_inputs(window)
    label = f"sink -inf, first tile below -128 log2 units, W={window}"
    say("case", label)
    gpu = run_gpu(inp, w.max_seqlen, scale, window)  # also asserts every value is finite
    check_full(gpu, _oracle_full(inp, scale, window), label)
    assert np.all(gpu["ds"] == 0.0)


def test_workload1_tiny_fp32_matches_oracle():
    w = WORKLOADS[1]
    say("case workload 1", w.name)
    inp = make_inputs(w)
    gpu = run_gpu(inp, w.max_seqlen, w.softmax_scale, w.window)
    ref = _oracle_full(inp, w.softmax_scale, w.window)
    errs = check_full(gpu, ref, w.name)
    errs["ds_head_max"] = _ds_head_max(gpu["ds"], ref["ds"])
    record_errors(w.name, "every element", errs)


def test_forward_is_deterministic_and_packing_is_invariant():
    w = custom_workload((130, 7, 64, 1), 8, 2, 64, 0, "bf16")
    inp = make_inputs(w, seed=99)
    say("case packing invariance", w.lengths)
    a = run_gpu(inp, w.max_seqlen, w.softmax_scale, 0)
    b = run_gpu(inp, w.max_seqlen, w.softmax_scale, 0)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])
    cu = inp["cu_seqlens"].numpy()
    ds_sum = np.zeros_like(a["ds"])
    for s in range(len(cu) - 1):
        sl = slice(int(cu[s]), int(cu[s + 1]))
        one = {n: inp[n][sl] for n in ("q", "k", "v", "dout")}
        one["sinks"] = inp["sinks"]
        one["cu_seqlens"] = torch.tensor([0, cu[s + 1] - cu[s]], dtype=torch.int32)
        r = run_gpu(one, int(cu[s + 1] - cu[s]), w.softmax_scale, 0)
        assert np.array_equal(r["o"], a["o"][sl])
        assert np.array_equal(r["lse"], a["lse"][:, sl])
        for n in ("dq", "dk", "dv"):
            assert max_abs(r[n], a[n][sl]) < 2e-2
        ds_sum += r["ds"]
    assert rel_l2(ds_sum, a["ds"]) < 1e-5


@pytest.mark.parametrize("heads", [1, 2, "group"])
@pytest.mark.parametrize("window", [0, 37])
def test_backward_is_bitwise_reproducible(monkeypatch, heads, window):
    """Same inputs, different workspace garbage: identical bits (no atomics)."""
    import attention_sink_fwd_amd as sa

    w = custom_workload((300, 5, 190), 8, 2, 64, window, "bf16")
    hg = 4 if heads == "group" else heads
    monkeypatch.setenv("SINK_ATTN_DKDV_HEADS", str(hg))
    say("case bitwise backward", w.lengths, "window", window, "dkdv_heads", hg)
    d = {k: v.to("cuda:0") for k, v in make_inputs(w, seed=5 + window).items()}
    o, lse = sa.sink_attn_fwd(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens"], w.max_seqlen,
                              w.softmax_scale, window)
    nb = sa.sink_attn_bwd_workspace_size(d["q"], d["k"], d["cu_seqlens"], w.max_seqlen,
                                         w.softmax_scale, window)
    outs = []
    for fill in (0x00, 0x7F):
        ws = torch.full((nb,), fill, dtype=torch.uint8, device="cuda:0")
        r = sa.sink_attn_bwd(d["q"], d["k"], d["v"], d["sinks"], o, lse, d["dout"], d["cu_seqlens"],
                             w.max_seqlen, w.softmax_scale, window, workspace=ws)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in r])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("lengths,hq,hkv,window,dtype", [
    ((300, 5, 190), 8, 2, 0, "bf16"),
    ((333, 129), 8, 1, 128, "bf16"),
    ((200, 70), 4, 2, 9, "f32"),
])
def test_forward_head_packing_keeps_every_bit(monkeypatch, lengths, hq, hkv, window, dtype):
    """Rows computed with several query heads per workgroup equal the rows
    computed one head per workgroup, bit for bit, and match the oracle."""
    import attention_sink_fwd_amd as sa

    w = custom_workload(lengths, hq, hkv, 64 if dtype == "bf16" else 40, window, dtype)
    inp = make_inputs(w, seed=41)
    d = {k: v.to("cuda:0") for k, v in inp.items()}
    outs = []
    for hp in (1, 2, hq // hkv):
        monkeypatch.setenv("SINK_ATTN_PACK_HEADS", str(hp))
        say("case head packing", lengths, "heads per workgroup", hp)
        outs.append(sa.sink_attn_fwd(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens"],
                                     w.max_seqlen, w.softmax_scale, window))
    torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])
    o_ref, lse_ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["cu_seqlens"],
                                    w.softmax_scale, window)
    assert max_abs(outs[-1][0].double().cpu().numpy(), o_ref) <= TOL_O
    assert max_abs(outs[-1][1].double().cpu().numpy(), lse_ref) <= TOL_LSE


@pytest.mark.parametrize("window", [0, 21])
def test_backward_head_packing_keeps_gradients(monkeypatch, window):
    """dQ, dK, dV do not depend on how many query heads a dQ workgroup packs
    (bit for bit); dS only through the order of its partial sums."""
    import attention_sink_fwd_amd as sa

    w = custom_workload((260, 3, 129), 8, 2, 64, window, "bf16")
    d = {k: v.to("cuda:0") for k, v in make_inputs(w, seed=8).items()}
    res = []
    for hp in (1, 2, 4):
        monkeypatch.setenv("SINK_ATTN_PACK_HEADS", str(hp))
        say("case backward packing", hp, "window", window)
        o, lse = sa.sink_attn_fwd(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens"], w.max_seqlen,
                                  w.softmax_scale, window)
        res.append(sa.sink_attn_bwd(d["q"], d["k"], d["v"], d["sinks"], o, lse, d["dout"],
                                    d["cu_seqlens"], w.max_seqlen, w.softmax_scale, window))
    torch.cuda.synchronize()
    for r in res[1:]:
        for a, b in zip(r[:3], res[0][:3]):
            assert torch.equal(a, b)
        assert rel_l2(r[3].double().cpu().numpy(), res[0][3].double().cpu().numpy()) < 1e-5


def test_autograd_wrapper_gives_the_entry_points_gradients():
    """torch autograd through sink_attention: O and every gradient equal the
    direct C-ABI calls bit for bit, and the oracle within tolerance."""
    import attention_sink_fwd_amd as sa

    w = custom_workload((150, 40), 8, 2, 64, 0, "bf16")
    inp = make_inputs(w, seed=77)
    say("case autograd wrapper", w.lengths)
    d = {k: v.to("cuda:0") for k, v in inp.items()}
    leaves = {n: d[n].clone().requires_grad_(True) for n in ("q", "k", "v", "sinks")}
    o = sa.sink_attention(leaves["q"], leaves["k"], leaves["v"], leaves["sinks"], d["cu_seqlens"],
                          w.max_seqlen)
    (o.float() * d["dout"].float()).sum().backward()
    o2, lse2 = sa.sink_attn_fwd(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens"], w.max_seqlen)
    dq, dk, dv, ds = sa.sink_attn_bwd(d["q"], d["k"], d["v"], d["sinks"], o2, lse2, d["dout"],
                                      d["cu_seqlens"], w.max_seqlen)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for name, ref in (("q", dq), ("k", dk), ("v", dv), ("sinks", ds)):
        assert torch.equal(leaves[name].grad, ref), name
    gpu = {"o": o2.double().cpu().numpy(), "lse": lse2.double().cpu().numpy(),
           "dq": dq.double().cpu().numpy(), "dk": dk.double().cpu().numpy(),
           "dv": dv.double().cpu().numpy(), "ds": ds.double().cpu().numpy()}
    check_full(gpu, _oracle_full(inp, w.softmax_scale, 0), "autograd wrapper")


def test_empty_batch_zeroes_dsinks():
    import attention_sink_fwd_amd as sa
    dev = "cuda:0"
    q = torch.empty((0, 4, 64), dtype=torch.bfloat16, device=dev)
    k = torch.empty((0, 2, 64), dtype=torch.bfloat16, device=dev)
    sinks = torch.randn(4, device=dev)
    cu = torch.zeros(3, dtype=torch.int32, device=dev)
    o, lse = sa.sink_attn_fwd(q, k, k, sinks, cu, 0)
    dsinks = torch.full((4,), 7.0, device=dev)
    sa.sink_attn_bwd(q, k, k, sinks, o, lse, o, cu, 0, dsinks=dsinks)
    torch.cuda.synchronize()
    assert torch.all(dsinks == 0).item()


# ---------------------------------------------------------------------------
# Full-size workloads (the shapes the benchmark times).


def _kv_group_reference(inp, scale, window, g, seqs=None):
    """Oracle restricted to KV group g (and optionally some sequences)."""
    q, k, v, do, s, cu = (inp[n] for n in ("q", "k", "v", "dout", "sinks", "cu_seqlens"))
    cu = cu.numpy()
    hq, hkv = q.shape[1], k.shape[1]
    grp = hq // hkv
    heads = list(range(g * grp, (g + 1) * grp))
    out = []
    for sidx in (range(len(cu) - 1) if seqs is None else seqs):
        b, e = int(cu[sidx]), int(cu[sidx + 1])
        c1 = np.array([0, e - b])
        sl = slice(b, e)
        o, lse = oracle.forward(q[sl], k[sl], v[sl], s, c1, scale, window, heads=heads)
        dq, dk, dv, ds = oracle.backward(q[sl], k[sl], v[sl], s, do[sl], c1, scale, window,
                                         kv_heads=[g])
        out.append((sidx, b, e, heads, o, lse, dq, dk, dv, ds))
    return out


def _check_group(gpu, refs, g, label):
    errs = {"o": 0.0, "lse": 0.0}
    num = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    den = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for (sidx, b, e, heads, o, lse, dq, dk, dv, ds) in refs:
        errs["o"] = max(errs["o"], max_abs(gpu["o"][b:e, heads], o[:, heads]))
        errs["lse"] = max(errs["lse"], max_abs(gpu["lse"][heads, b:e], lse[heads]))
        for n, ref, got in (("dq", dq[:, heads], gpu["dq"][b:e, heads]),
                            ("dk", dk[:, g], gpu["dk"][b:e, g]),
                            ("dv", dv[:, g], gpu["dv"][b:e, g])):
            num[n] += float(np.sum((got - ref) ** 2))
            den[n] += float(np.sum(ref ** 2))
    for n in num:
        errs[n] = math.sqrt(num[n] / den[n])
    say(f"  {label} group {g}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for n in den:
        errs["_den_" + n] = den[n]
    assert errs["o"] <= TOL_O and errs["lse"] <= TOL_LSE, errs
    assert errs["dq"] <= TOL_GRAD and errs["dk"] <= TOL_GRAD and errs["dv"] <= TOL_GRAD, errs
    return errs


def _ds_head_max(got, ref):
    """Largest per-head relative error of dS (heads whose exact |dS| is below
    1e-6 count with their absolute error)."""
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-6)))


def _ds_self_consistency(gpu, inp):
    """dS_h == -sum_i exp(S_h - LSE_i) (dO_i . O_i) on the GPU's own O and LSE."""
    s = inp["sinks"].double().numpy()
    do = inp["dout"].double().numpy()
    dvec = np.einsum("thd,thd->ht", do, gpu["o"])
    want = -np.sum(np.exp(s[:, None] - gpu["lse"]) * dvec, axis=1)
    return rel_l2(gpu["ds"], want)


@pytest.mark.parametrize("window", [0, 128])
def test_maximum_size_batch_against_oracle(window):
    """The largest batch the boundary accepts at the GPT-OSS head shape:
    T * Hq * d = 2^31 - 4096 elements (127 sequences of 4096 tokens and one
    of 4095, 64 query heads, 8 KV heads, d = 64), where element offsets into
    Q, O, dO and dQ come within one row of 2^31.  The last sequence's last KV
    group (the largest offsets) against the oracle, every row and key; dS of
    every head through the identity dS_h = -sum_i exp(S_h - LSE_i) dO_i . O_i
    on the GPU's own O and LSE (float64 on the device)."""
    import attention_sink_fwd_amd as sa

    lengths = (4096,) * 127 + (4095,)
    w = custom_workload(lengths, 64, 8, 64, window, "bf16", name="max_size")
    assert w.total_tokens * 64 * 64 == 2 ** 31 - 4096
    say("case maximum size", w.total_tokens, "tokens, window", window)
    dev = "cuda:0"
    d = make_inputs_device(w, seed=31 + window, device=dev)
    o, lse = sa.sink_attn_fwd(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens"], w.max_seqlen,
                              w.softmax_scale, window)
    dq, dk, dv, ds = sa.sink_attn_bwd(d["q"], d["k"], d["v"], d["sinks"], o, lse, d["dout"],
                                      d["cu_seqlens"], w.max_seqlen, w.softmax_scale, window)
    torch.cuda.synchronize()
    for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv), ("ds", ds)):
        assert bool(torch.isfinite(t).all()), name
    # dS of every head from the GPU's own O and LSE, chunked over tokens.
    want = torch.zeros(64, dtype=torch.float64, device=dev)
    s64 = d["sinks"].double()
    for r in range(0, w.total_tokens, 1 << 16):
        e = min(r + (1 << 16), w.total_tokens)
        dvec = (d["dout"][r:e].double() * o[r:e].double()).sum(-1)  # [rows, Hq]
        want -= (torch.exp(s64[None, :] - lse[:, r:e].double().T) * dvec).sum(0)
    e_ds = rel_l2(ds.double().cpu().numpy(), want.cpu().numpy())
    # The last sequence, KV group 7, against the oracle.
    b = w.total_tokens - lengths[-1]
    host = {n: d[n][b:].cpu() for n in ("q", "k", "v", "dout")}
    host["sinks"], host["cu_seqlens"] = d["sinks"].cpu(), torch.tensor([0, lengths[-1]], dtype=torch.int32)
    gpu = {"o": f64(o[b:]), "lse": f64(lse[:, b:]), "dq": f64(dq[b:]), "dk": f64(dk[b:]),
           "dv": f64(dv[b:]), "ds": f64(ds)}
    refs = _kv_group_reference(host, w.softmax_scale, window, 7)
    errs = _check_group(gpu, refs, 7, f"maximum size, window {window}")
    say(f"  dS identity over all heads: {e_ds:.2e}")
    assert e_ds <= TOL_DS


@pytest.mark.parametrize("wid", [2, 3])
def test_full_workload_whole_kv_groups(wid):
    """Workloads 2 and 3: two whole KV groups against the oracle; dS in full."""
    w = WORKLOADS[wid]
    say("case workload", wid, w.name)
    inp = make_inputs(w)
    gpu = run_gpu(inp, w.max_seqlen, w.softmax_scale, w.window)
    hq, hkv = w.num_q_heads, w.num_kv_heads
    ds_ref = np.zeros(hq)
    ds_heads = []
    group_errs = []
    for g in (0, hkv - 3):
        refs = _kv_group_reference(inp, w.softmax_scale, w.window, g)
        group_errs.append(_check_group(gpu, refs, g, w.name))
        for r in refs:
            ds_ref[r[3]] += r[9][r[3]]
        ds_heads += r[3]
    a, b = group_errs
    e = rel_l2(gpu["ds"][ds_heads], ds_ref[ds_heads])
    say(f"  dS over heads {ds_heads[0]}..: {e:.2e}; self-consistency {_ds_self_consistency(gpu, inp):.2e}")
    assert e <= TOL_DS
    errs = {n: max(a[n], b[n]) for n in ("o", "lse")}
    errs.update({n: math.sqrt((a[n] ** 2 * a["_den_" + n] + b[n] ** 2 * b["_den_" + n]) /
                              (a["_den_" + n] + b["_den_" + n])) for n in ("dq", "dk", "dv")})
    errs["ds"] = e
    errs["ds_head_max"] = _ds_head_max(gpu["ds"][ds_heads], ds_ref[ds_heads])
    record_errors(w.name, f"KV groups 0 and {hkv - 3} (query heads {ds_heads[0]}-{ds_heads[7]}, "
                  f"{ds_heads[8]}-{ds_heads[-1]}), every row and key", errs)
    if wid == 2:
        _record_scaled_operand_share(inp, w, gpu)


def _rounded_operand(t, scale):
    """The score operand the kernels keep in registers, mapped back to the
    input's scale: bf16(t * scale * log2 e) / (scale * log2 e), with the
    factor formed in float32 as the library does."""
    c = np.float32(np.float32(scale) * np.float32(1.4426950408889634))
    x = (t.float() * float(c)).to(torch.bfloat16).double() / float(c)
    return x


def _record_scaled_operand_share(inp, w, gpu):
    """How far the oracle's own outputs move (KV group 0) when q, or k, is
    replaced everywhere by the bf16-rounded scaled operand the forward and
    dQ kernels (q) or the dK/dV kernel (k) multiply with, next to the GPU's
    total error on the same outputs."""
    g, grp = 0, w.num_q_heads // w.num_kv_heads
    heads = list(range(g * grp, (g + 1) * grp))
    exact = _kv_group_reference(inp, w.softmax_scale, w.window, g)[0]
    rows = {}
    for name in ("q", "k"):
        alt = dict(inp)
        alt[name] = _rounded_operand(inp[name], w.softmax_scale)
        r = _kv_group_reference(alt, w.softmax_scale, w.window, g)[0]
        rows[name] = {
            "o": max_abs(r[4][:, heads], exact[4][:, heads]),
            "lse": max_abs(r[5][heads], exact[5][heads]),
            "dq": rel_l2(r[6][:, heads], exact[6][:, heads]),
            "dk": rel_l2(r[7][:, g], exact[7][:, g]),
            "dv": rel_l2(r[8][:, g], exact[8][:, g]),
            "ds": rel_l2(r[9][heads], exact[9][heads]),
        }
    total = {
        "o": max_abs(gpu["o"][:, heads], exact[4][:, heads]),
        "lse": max_abs(gpu["lse"][heads], exact[5][heads]),
        "dq": rel_l2(gpu["dq"][:, heads], exact[6][:, heads]),
        "dk": rel_l2(gpu["dk"][:, g], exact[7][:, g]),
        "dv": rel_l2(gpu["dv"][:, g], exact[8][:, g]),
        "ds": rel_l2(gpu["ds"][heads], exact[9][heads]),
    }
    for name, vals in (("oracle, q -> bf16(q scale log2e)", rows["q"]),
                       ("oracle, k -> bf16(k scale log2e)", rows["k"]), ("GPU", total)):
        say(f"  KV group 0, {name}: " + " ".join(f"{k}={v:.2e}" for k, v in vals.items()))
        record_errors(w.name, f"KV group 0 (query heads 0-7): {name}, against the exact oracle", vals)


def test_full_workload4_long_context_sampled():
    """L = 65536 head share against the oracle: sampled rows (O, LSE, dQ) of
    four heads; dK, dV of one whole KV group (8 query heads) at keys 0-127
    (reductions over all 65536 rows), a middle tile and the last keys; dS of
    those 8 heads (every row)."""
    w = WORKLOADS[4]
    say("case workload 4", w.name)
    inp = make_inputs(w)
    gpu = run_gpu(inp, w.max_seqlen, w.softmax_scale, 0)
    L = w.max_seqlen
    rng = np.random.default_rng(404)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 4095, 4096, 32767, L - 2, L - 1],
                                     rng.integers(0, L, 13)]))
    q, k, v, do, s, cu = (inp[n] for n in ("q", "k", "v", "dout", "sinks", "cu_seqlens"))
    e_o = e_l = 0.0
    num = den = 0.0
    for h in (0, 7, 8, 15):
        o_r, l_r = oracle.forward_rows(q, k, v, s, cu, w.softmax_scale, 0, 0, h, rows)
        e_o = max(e_o, max_abs(gpu["o"][rows, h], o_r))
        e_l = max(e_l, max_abs(gpu["lse"][h, rows], l_r))
        dq_r = oracle.backward_rows(q, k, v, s, do, cu, w.softmax_scale, 0, 0, h, rows)
        num += float(np.sum((gpu["dq"][rows, h] - dq_r) ** 2))
        den += float(np.sum(dq_r ** 2))
    e_dq = math.sqrt(num / den)
    say(f"  sampled rows: o={e_o:.2e} lse={e_l:.2e} dq={e_dq:.2e}")
    # KV group 0: keys 0-127, 32768-32895 and the last 100 keys, every row of
    # its 8 query heads
    keys = np.concatenate([np.arange(128), np.arange(32768, 32896), np.arange(L - 100, L)])
    dk_r, dv_r, ds_g = oracle.backward_keys_blocked(q, k, v, s, do, cu, w.softmax_scale, 0, 0, 0, keys)
    blocks = {"keys 0-127": slice(0, 128), "keys 32768-32895": slice(128, 256), "last 100 keys": slice(256, None)}
    for name, sl in blocks.items():
        say(f"  {name}: dk={rel_l2(gpu['dk'][keys[sl], 0], dk_r[sl]):.2e} "
            f"dv={rel_l2(gpu['dv'][keys[sl], 0], dv_r[sl]):.2e}")
    e_dk, e_dv = rel_l2(gpu["dk"][keys, 0], dk_r), rel_l2(gpu["dv"][keys, 0], dv_r)
    heads = sorted(ds_g)
    ds_ref = np.array([ds_g[h] for h in heads])
    e_ds = rel_l2(gpu["ds"][heads], ds_ref)
    e_ds_head = _ds_head_max(gpu["ds"][heads], ds_ref)
    say(f"  o={e_o:.2e} lse={e_l:.2e} dq={e_dq:.2e} dk={e_dk:.2e} dv={e_dv:.2e} ds={e_ds:.2e} "
        f"(worst head {e_ds_head:.2e}); ds self-consistency {_ds_self_consistency(gpu, inp):.2e}")
    assert e_o <= TOL_O and e_l <= TOL_LSE
    assert e_dq <= TOL_GRAD and e_dk <= TOL_GRAD and e_dv <= TOL_GRAD
    for sl in blocks.values():
        assert rel_l2(gpu["dk"][keys[sl], 0], dk_r[sl]) <= TOL_GRAD
        assert rel_l2(gpu["dv"][keys[sl], 0], dv_r[sl]) <= TOL_GRAD
    assert e_ds <= TOL_DS
    record_errors(w.name, "O, LSE, dQ: 24 sampled rows of query heads 0, 7, 8, 15; dK, dV: KV group 0 at keys "
                  "0-127, 32768-32895 and the last 100; dS: query heads 0-7 (every row)",
                  {"o": e_o, "lse": e_l, "dq": e_dq, "dk": e_dk, "dv": e_dv, "ds": e_ds, "ds_head_max": e_ds_head})


def test_full_workload5_varlen_sampled_sequences():
    """64 packed sequences: whole KV groups of four sequences (incl. the
    shortest and longest) against the oracle, and dS of two heads over all
    64 sequences."""
    w = WORKLOADS[5]
    say("case workload 5", w.name)
    inp = make_inputs(w)
    gpu = run_gpu(inp, w.max_seqlen, w.softmax_scale, 0)
    lens = np.array(w.lengths)
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 2, 63})
    group_errs = []
    for g in (1, 6):
        refs = _kv_group_reference(inp, w.softmax_scale, 0, g, seqs=seqs)
        group_errs.append(_check_group(gpu, refs, g, w.name))
    q, k, v, do, s, cu = (inp[n] for n in ("q", "k", "v", "dout", "sinks", "cu_seqlens"))
    heads = [9, 50]
    ds_ref = np.zeros(len(heads))
    grp = w.num_q_heads // w.num_kv_heads
    for n, h in enumerate(heads):
        # head h alone (a one-head problem with its KV head), converted once
        sub = [t[:, h:h + 1].double().numpy() for t in (q, do)]
        kv = [t[:, h // grp:h // grp + 1].double().numpy() for t in (k, v)]
        for seq in range(len(lens)):
            _, _, part = oracle.backward_keys_blocked(sub[0], kv[0], kv[1], s[h:h + 1], sub[1], cu,
                                                      w.softmax_scale, 0, seq, 0, [])
            ds_ref[n] += part[0]
    e_ds = rel_l2(gpu["ds"][heads], ds_ref)
    e_ds_head = _ds_head_max(gpu["ds"][heads], ds_ref)
    say(f"  dS heads {heads}: {e_ds:.2e} (worst head {e_ds_head:.2e}); self-consistency "
        f"{_ds_self_consistency(gpu, inp):.2e}")
    assert e_ds <= TOL_DS
    a, b = group_errs
    errs = {n: max(a[n], b[n]) for n in ("o", "lse")}
    errs.update({n: math.sqrt((a[n] ** 2 * a["_den_" + n] + b[n] ** 2 * b["_den_" + n]) /
                              (a["_den_" + n] + b["_den_" + n])) for n in ("dq", "dk", "dv")})
    errs["ds"] = e_ds
    errs["ds_head_max"] = e_ds_head
    record_errors(w.name, f"O, LSE, dQ, dK, dV: KV groups 1 and 6 over sequences {seqs} (every row and key); "
                  f"dS: query heads {heads} over all 64 sequences", errs)
