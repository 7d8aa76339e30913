"""Short sliding windows (1..128 keys, bf16, head_dim 64): the fused backward
kernel (one workgroup per run of 1 to 4 consecutive 128-row query tiles and
KV group; dQ, dK, dV and the sink gradient from one pass) and, with
SINK_ATTN_BWD_FUSED=0, the dQ and dK/dV kernels, each against the float64
oracle on every element.

Shapes cover one-row and one-step tiles, a last tile of one row, windows of
1, 63, 64, 127 and 128 keys, empty and mixed-length sequences, query heads
per KV head 1, 3, 4, 8 and 64, and sinks of -inf, +30 and mixed values.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synthetic.workloads import custom_workload, make_inputs
from tests.parity_util import check_full, rel_l2, run_gpu, say
from tests.test_gpu_parity import _oracle_full, _set_sinks

pytestmark = pytest.mark.gpu

CASES = [
    # lengths, hq, hkv, window, sinks
    ((2,), 4, 2, 1, "normal"),
    ((64,), 8, 1, 63, "normal"),
    ((65,), 8, 2, 64, "mixed"),
    ((128,), 2, 1, 127, "normal"),
    ((129,), 4, 1, 128, "normal"),
    ((257, 3, 200, 0, 130), 8, 2, 128, "normal"),
    ((700,), 16, 2, 100, "mixed"),
    ((390, 260), 6, 2, 33, "normal"),
    ((300,), 64, 1, 128, "normal"),
    ((250,), 8, 8, 128, "minus_inf"),
    ((190,), 4, 2, 50, "plus30"),
    ((1000,), 8, 2, 1, "normal"),
    # workgroups take two 128-row tiles: one whole pair, a pair and a single
    # tile, two pairs, and a pair whose second tile has one row
    ((256,), 8, 2, 128, "normal"),
    ((384, 512), 4, 1, 100, "mixed"),
    ((257, 385), 8, 2, 128, "normal"),
]


@pytest.mark.parametrize("path", ["fused", "two_kernel"])
@pytest.mark.parametrize("lengths,hq,hkv,window,sinks", CASES)
def test_short_window_matches_oracle(monkeypatch, path, lengths, hq, hkv, window, sinks):
    monkeypatch.setenv("SINK_ATTN_BWD_FUSED", "1" if path == "fused" else "0")
    label = f"{path} L={lengths} hq={hq} hkv={hkv} W={window} sinks={sinks}"
    say("case", label)
    w = custom_workload(lengths, hq, hkv, 64, window, "bf16")
    inp = _set_sinks(make_inputs(w, seed=sum(lengths) + 3 * hq + window), sinks, hq)
    scale = 1.0 / math.sqrt(64)
    gpu = run_gpu(inp, w.max_seqlen, scale, window)
    check_full(gpu, _oracle_full(inp, scale, window), label)
    if sinks == "minus_inf":
        assert np.all(gpu["ds"] == 0.0)


@pytest.mark.parametrize("tiles", ["1", "2", "3", "4"])
@pytest.mark.parametrize("lengths,hq,hkv,window", [
    ((1000, 257, 130), 8, 2, 128),  # 8, 3 and 2 tiles: ragged last runs, a last tile of one or two rows
    ((640, 1), 4, 1, 100),          # 5 tiles, then a one-token sequence
    ((900,), 16, 2, 33),
])
def test_fused_tiles_per_workgroup_match_oracle(monkeypatch, tiles, lengths, hq, hkv, window):
    """Every number of query tiles per fused workgroup (SINK_ATTN_FUSED_TILES)
    against the oracle: the key tiles shared between runs go through the two
    float planes, the others are written whole."""
    monkeypatch.setenv("SINK_ATTN_BWD_FUSED", "1")
    monkeypatch.setenv("SINK_ATTN_FUSED_TILES", tiles)
    label = f"fused tiles {tiles} L={lengths} hq={hq} hkv={hkv} W={window}"
    say("case", label)
    w = custom_workload(lengths, hq, hkv, 64, window, "bf16")
    inp = make_inputs(w, seed=sum(lengths) + int(tiles))
    gpu = run_gpu(inp, w.max_seqlen, w.softmax_scale, window)
    check_full(gpu, _oracle_full(inp, w.softmax_scale, window), label)


def test_fused_and_two_kernel_paths_agree(monkeypatch):
    """The two paths score with the same bf16 operands and differ only in
    float summation order: their outputs agree far inside the oracle
    tolerance, and the forward outputs they start from are identical."""
    w = custom_workload((600, 333), 8, 2, 64, 128, "bf16")
    inp = make_inputs(w, seed=4242)
    say("case paths agree", w.lengths)
    res = {}
    for path in ("1", "0"):
        monkeypatch.setenv("SINK_ATTN_BWD_FUSED", path)
        res[path] = run_gpu(inp, w.max_seqlen, w.softmax_scale, 128)
    assert np.array_equal(res["1"]["o"], res["0"]["o"])
    for n in ("dq", "dk", "dv", "ds"):
        e = rel_l2(res["1"][n], res["0"][n])
        say(f"  {n} fused vs two-kernel rel-L2 {e:.2e}")
        assert e < 5e-3, (n, e)


def test_fused_backward_is_bitwise_reproducible_at_scale(monkeypatch):
    """Two 4096-token sequences, 64 query heads on 8 KV heads, window 128:
    256 fused workgroups at once, three runs over different workspace
    contents give identical bits.  Each of the kernel's producer wavefronts
    forms the statistics of the rows it loaded itself; a hand-over between
    wavefronts without a barrier would show here as run-to-run differences."""
    import attention_sink_fwd_amd as sa

    monkeypatch.setenv("SINK_ATTN_BWD_FUSED", "1")
    w = custom_workload((4096, 4096), 64, 8, 64, 128, "bf16")
    say("case fused bitwise at scale", w.lengths)
    d = {k: v.to("cuda:0") for k, v in make_inputs(w, seed=77).items()}
    assert sa.sink_attn_bwd_fused(d["q"], d["k"], d["cu_seqlens"], w.max_seqlen, w.softmax_scale, 128)
    o, lse = sa.sink_attn_fwd(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens"], w.max_seqlen,
                              w.softmax_scale, 128)
    nb = sa.sink_attn_bwd_workspace_size(d["q"], d["k"], d["cu_seqlens"], w.max_seqlen, w.softmax_scale, 128)
    outs = []
    for fill in (0x00, 0x7F, 0xFF):
        ws = torch.full((nb,), fill, dtype=torch.uint8, device="cuda:0")
        r = sa.sink_attn_bwd(d["q"], d["k"], d["v"], d["sinks"], o, lse, d["dout"], d["cu_seqlens"],
                             w.max_seqlen, w.softmax_scale, 128, workspace=ws)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in r])
    for run in outs[1:]:
        for a, b in zip(outs[0], run):
            assert torch.equal(a, b)
    # and the first run is right: dS_h against its definition on the GPU's own O and LSE
    s = d["sinks"].double().cpu()
    dvec = torch.einsum("thd,thd->ht", d["dout"].double().cpu(), o.double().cpu())
    want = -(torch.exp(s[:, None] - lse.double().cpu()) * dvec).sum(dim=1)
    assert rel_l2(outs[0][3].double().cpu().numpy(), want.numpy()) < 1e-5
