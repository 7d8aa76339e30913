"""Paged-cache forward (prefill and decode) on the GPU, through the C ABI.

Against the float64 oracle (``oracle.forward_paged``) element by element, and
bit for bit against the training forward's rows at the same positions.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synthetic.workloads import custom_workload, make_inputs, make_paged
from tests.parity_util import TOL_LSE, TOL_O, max_abs, say

pytestmark = pytest.mark.gpu

CASES = [
    # lengths (keys per sequence), new tokens per sequence, hq, hkv, d, window, dtype, page size
    ((130, 5, 257), (1, 5, 64), 8, 2, 64, 0, "bf16", 64),
    ((300, 1, 64, 65, 700), (1, 1, 1, 1, 1), 8, 2, 64, 0, "bf16", 128),
    ((333, 129), (100, 2), 4, 1, 64, 48, "bf16", 64),
    ((200, 70), (7, 70), 4, 2, 40, 0, "f32", 64),
    ((190, 64), (33, 64), 4, 2, 16, 0, "bf16", 256),
    # both sides of the 32-key / 64-key tile boundary at window 128
    ((700, 300), (1, 120), 16, 2, 64, 128, "bf16", 64),
    ((700, 300), (1, 120), 16, 2, 64, 129, "bf16", 128),
    ((500, 90), (60, 1), 4, 2, 40, 32, "f32", 64),
]


def _run(pg, w, dev="cuda:0"):
    import attention_sink_fwd_amd as sa

    d = {k: v.to(dev) for k, v in pg.items() if k != "rows"}
    ql = np.diff(pg["cu_seqlens"].numpy())
    o, lse = sa.sink_attn_fwd_paged(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                    d["kv_lens"], d["sinks"], d["cu_seqlens"], int(ql.max()),
                                    w.softmax_scale, w.window)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("lengths,q_lens,hq,hkv,d,window,dtype,ps", CASES)
def test_paged_forward_matches_oracle(lengths, q_lens, hq, hkv, d, window, dtype, ps):
    label = f"L={lengths} new={q_lens} hq={hq} hkv={hkv} d={d} W={window} {dtype} page={ps}"
    say("case", label)
    w = custom_workload(lengths, hq, hkv, d, window, dtype)
    inp = make_inputs(w, seed=sum(lengths) + d)
    pg = make_paged(inp, q_lens, ps, seed=7)
    o, lse = _run(pg, w)
    o_ref, lse_ref = oracle.forward_paged(pg["q"], pg["k_cache"], pg["v_cache"], pg["block_table"],
                                          pg["kv_lens"], pg["sinks"], pg["cu_seqlens"],
                                          w.softmax_scale, window)
    eo, el = max_abs(o.double().cpu().numpy(), o_ref), max_abs(lse.double().cpu().numpy(), lse_ref)
    say(f"  errors: o={eo:.2e} lse={el:.2e}")
    assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.parametrize("fwd_heads", [None, 1, 2])
@pytest.mark.parametrize("lengths,q_lens,hq,hkv,d,window,dtype,ps", CASES)
def test_paged_forward_is_bit_identical_to_training_rows(monkeypatch, fwd_heads, lengths, q_lens,
                                                         hq, hkv, d, window, dtype, ps):
    import attention_sink_fwd_amd as sa

    if fwd_heads is not None:
        if (hq // hkv) % fwd_heads:
            pytest.skip("head count does not divide the group")
        # the same packing for both calls; None: each call's own default
        monkeypatch.setenv("SINK_ATTN_PACK_HEADS", str(fwd_heads))
    say("case bits", lengths, q_lens, d, window, dtype, ps, "fwd_heads", fwd_heads)
    w = custom_workload(lengths, hq, hkv, d, window, dtype)
    inp = make_inputs(w, seed=sum(lengths) + 3 * d)
    dev = {k: v.to("cuda:0") for k, v in inp.items()}
    o_t, lse_t = sa.sink_attn_fwd(dev["q"], dev["k"], dev["v"], dev["sinks"], dev["cu_seqlens"],
                                  w.max_seqlen, w.softmax_scale, window)
    pg = make_paged(inp, q_lens, ps, seed=13)
    o, lse = _run(pg, w)
    rows = pg["rows"].to("cuda:0")
    assert torch.equal(o, o_t[rows])
    assert torch.equal(lse, lse_t[:, rows])


def test_paged_decode_full_size_bits_and_sampled_oracle():
    """GPT-OSS attention shape, 16 sequences of 1000-6000 cached keys, one new
    token each: bit-identical to the training forward's last rows, and a few
    heads against the oracle."""
    import attention_sink_fwd_amd as sa

    lengths = tuple(int(x) for x in np.random.default_rng(21).integers(1000, 6000, size=16))
    w = custom_workload(lengths, 64, 8, 64, 0, "bf16")
    say("case full-size decode", lengths)
    inp = make_inputs(w, seed=21)
    dev = {k: v.to("cuda:0") for k, v in inp.items()}
    o_t, lse_t = sa.sink_attn_fwd(dev["q"], dev["k"], dev["v"], dev["sinks"], dev["cu_seqlens"],
                                  w.max_seqlen, w.softmax_scale, 0)
    pg = make_paged(inp, (1,) * 16, 64, seed=5)
    o, lse = _run(pg, w)
    rows = pg["rows"].to("cuda:0")
    assert torch.equal(o, o_t[rows]) and torch.equal(lse, lse_t[:, rows])
    # oracle on two KV groups' worth of heads, all 16 new tokens
    sub = {k: v for k, v in pg.items()}
    heads = [0, 1, 9, 63]
    sub["q"] = pg["q"][:, heads]
    sub["sinks"] = pg["sinks"][heads]
    # keep the query -> KV head mapping of the full problem: heads 0, 1 -> g0, 9 -> g1, 63 -> g7
    kv_heads = [0, 0, 1, 7]
    sub["k_cache"] = pg["k_cache"][:, :, kv_heads]
    sub["v_cache"] = pg["v_cache"][:, :, kv_heads]
    o_ref, lse_ref = oracle.forward_paged(sub["q"], sub["k_cache"], sub["v_cache"], sub["block_table"],
                                          sub["kv_lens"], sub["sinks"], sub["cu_seqlens"],
                                          w.softmax_scale, 0)
    got_o = o[:, heads].double().cpu().numpy()
    got_l = lse[heads].double().cpu().numpy()
    assert max_abs(got_o, o_ref) <= TOL_O and max_abs(got_l, lse_ref) <= TOL_LSE


@pytest.mark.parametrize("d,window,dtype", [(64, 0, "bf16"), (64, 500, "bf16"), (40, 0, "f32")])
def test_long_sequence_forward_bits_and_sampled_oracle(d, window, dtype):
    """A batch whose longest sequence reaches 16384 tokens runs the training
    forward with eight wavefronts per workgroup (the paged forward keeps
    four): the rows must still match the paged forward bit for bit, and
    sampled rows the oracle."""
    import attention_sink_fwd_amd as sa

    lengths, q_lens = (16400, 37, 0, 130), (300, 37, 0, 130)
    w = custom_workload(lengths, 4, 2, d, window, dtype)
    say("case long forward", lengths, d, window, dtype)
    inp = make_inputs(w, seed=16400 + d + window)
    dev = {k: v.to("cuda:0") for k, v in inp.items()}
    o_t, lse_t = sa.sink_attn_fwd(dev["q"], dev["k"], dev["v"], dev["sinks"], dev["cu_seqlens"],
                                  w.max_seqlen, w.softmax_scale, window)
    pg = make_paged(inp, q_lens, 64, seed=17)
    o, lse = _run(pg, w)
    rows = pg["rows"].to("cuda:0")
    assert torch.equal(o, o_t[rows]) and torch.equal(lse, lse_t[:, rows])
    sample = np.array([0, 1, 63, 64, 255, 256, 8191, 16383, 16384, 16398, 16399])
    got_o = o_t.double().cpu().numpy()
    got_l = lse_t.double().cpu().numpy()
    e_o = e_l = 0.0
    for h in (0, 3):
        o_r, l_r = oracle.forward_rows(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["cu_seqlens"],
                                       w.softmax_scale, window, 0, h, sample)
        e_o = max(e_o, max_abs(got_o[sample, h], o_r))
        e_l = max(e_l, max_abs(got_l[h, sample], l_r))
    # the short sequences of the same launch, every element
    cu = inp["cu_seqlens"].numpy()
    for sq in (1, 3):
        b, e = int(cu[sq]), int(cu[sq + 1])
        c1 = np.array([0, e - b])
        o_r, l_r = oracle.forward(inp["q"][b:e], inp["k"][b:e], inp["v"][b:e], inp["sinks"], c1,
                                  w.softmax_scale, window)
        e_o = max(e_o, max_abs(got_o[b:e], o_r))
        e_l = max(e_l, max_abs(got_l[:, b:e], l_r))
    say(f"  sampled rows and short sequences: o={e_o:.2e} lse={e_l:.2e}")
    assert e_o <= TOL_O and e_l <= TOL_LSE


@pytest.mark.parametrize("factor", [8.0, 80.0])
def test_paged_rows_bit_identical_under_large_logit_jumps(factor):
    """The forward's raise decisions (integer shifts, exact-maximum path on an
    overflowing tile) depend on each row alone: paged rows equal the
    training rows bit for bit on inputs that trigger both."""
    import attention_sink_fwd_amd as sa
    from tests.test_gpu_parity import large_logit_inputs

    w, inp, scale = large_logit_inputs(factor, 0)
    say("case paged large logits", factor)
    dev = {k: v.to("cuda:0") for k, v in inp.items()}
    o_t, lse_t = sa.sink_attn_fwd(dev["q"], dev["k"], dev["v"], dev["sinks"], dev["cu_seqlens"],
                                  w.max_seqlen, scale, 0)
    pg = make_paged(inp, (180, 77), 64, seed=19)
    d = {k: v.to("cuda:0") for k, v in pg.items() if k != "rows"}
    o, lse = sa.sink_attn_fwd_paged(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["kv_lens"],
                                    d["sinks"], d["cu_seqlens"], 180, scale, 0)
    torch.cuda.synchronize()
    rows = pg["rows"].to("cuda:0")
    assert torch.isfinite(o_t).all() and torch.isfinite(lse_t).all()
    assert torch.equal(o, o_t[rows]) and torch.equal(lse, lse_t[:, rows])


@pytest.mark.parametrize("window", [0, 40])
def test_paged_rows_bit_identical_with_minus_inf_sink_and_very_negative_scores(window):
    """Sink -inf and a first key tile scoring about -160 log2 units: the
    paged rows equal the training rows bit for bit and are finite."""
    import attention_sink_fwd_amd as sa
    from tests.test_gpu_parity import very_negative_first_tile_inputs

    w, inp, scale = very_negative_first_tile_inputs(window)
    say("case paged, sink -inf, very negative first tile, window", window)
    dev = {k: v.to("cuda:0") for k, v in inp.items()}
    o_t, lse_t = sa.sink_attn_fwd(dev["q"], dev["k"], dev["v"], dev["sinks"], dev["cu_seqlens"],
                                  w.max_seqlen, scale, window)
    pg = make_paged(inp, (180, 77), 64, seed=23)
    d = {k: v.to("cuda:0") for k, v in pg.items() if k != "rows"}
    o, lse = sa.sink_attn_fwd_paged(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["kv_lens"],
                                    d["sinks"], d["cu_seqlens"], 180, scale, window)
    torch.cuda.synchronize()
    rows = pg["rows"].to("cuda:0")
    assert torch.isfinite(o_t).all() and torch.isfinite(lse_t).all()
    assert torch.equal(o, o_t[rows]) and torch.equal(lse, lse_t[:, rows])


def _draw_paged_shape(seed):
    rng = np.random.default_rng(seed)
    nseq = int(rng.integers(1, 9))
    lens = [int(x) for x in rng.integers(1, 3000, size=nseq)]
    decode = rng.random() < 0.5
    q_lens = [1 if decode else int(rng.integers(1, L + 1)) for L in lens]
    hkv = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * int(rng.choice([1, 2, 4, 8, 16]))
    d = int(rng.choice([64, 64, 64, 32, 40]))
    dtype = "bf16" if rng.random() < 0.85 else "f32"
    window = 0 if rng.random() < 0.5 else int(rng.integers(1, 400))
    ps = int(rng.choice([64, 128, 256, 512]))
    sinks = str(rng.choice(["normal", "mixed", "minus_inf"]))
    return lens, q_lens, hq, hkv, d, dtype, window, ps, sinks


@pytest.mark.parametrize("seed", range(7000, 7040))
def test_random_paged_shapes_bit_identical_to_training_rows(seed):
    """Seeded random batches: one to eight sequences of 1..2999 cached keys,
    decode (one new token each) or prefill (1..L new tokens), pages of 64 to
    512 keys in shuffled order (unused slots hold NaN), windows, float32 and
    head dimensions 32 to 64.  The new rows equal the training forward's rows
    at the same positions bit for bit, and are finite."""
    import attention_sink_fwd_amd as sa
    from tests.test_gpu_parity import _set_sinks

    lens, q_lens, hq, hkv, d, dtype, window, ps, sinks = _draw_paged_shape(seed)
    say("case paged random", seed, lens, "decode" if max(q_lens) == 1 else "prefill", hq, hkv, d, dtype,
        window, ps, sinks)
    w = custom_workload(lens, hq, hkv, d, window, dtype)
    inp = _set_sinks(make_inputs(w, seed=seed), sinks, hq)
    dev = {k: v.to("cuda:0") for k, v in inp.items()}
    o_t, lse_t = sa.sink_attn_fwd(dev["q"], dev["k"], dev["v"], dev["sinks"], dev["cu_seqlens"],
                                  w.max_seqlen, w.softmax_scale, window)
    pg = make_paged(inp, q_lens, ps, seed=seed)
    o, lse = _run(pg, w)
    rows = pg["rows"].to("cuda:0")
    assert torch.isfinite(o).all()
    assert torch.equal(o, o_t[rows]) and torch.equal(lse, lse_t[:, rows])
