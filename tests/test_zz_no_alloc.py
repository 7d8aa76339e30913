"""sink_attn_bwd_noalloc through the C ABI against sink_attn_bwd.

Two calls in a row on one device, the second with a smaller input, so the
second runs on the buffer the first left behind.  The first shape (GPT-OSS
attention, 4096 tokens) needs more workspace than the buffer holds with
sink_attn_bwd's split, so the no-allocation call takes more query heads per
dK/dV workgroup: dQ and dS are bitwise identical, dK and dV differ only in
the order of their float additions.  The second shape fits with the same
split: every output bitwise identical.
"""
import ctypes

import numpy as np
import pytest
import torch

from attention_sink_fwd_amd import _lib
from synthetic.workloads import WORKLOADS, custom_workload, make_inputs
from tests.parity_util import TOL_DS, TOL_GRAD, f64, rel_l2, say

pytestmark = pytest.mark.gpu


def _call_noalloc(d, w, window):
    import attention_sink_fwd_amd as sa

    lib = _lib.load()
    q, k = d["q"], d["k"]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    ds = torch.empty_like(d["sinks"])
    p = sa.make_params(q, k, d["cu_seqlens"], w.max_seqlen, w.softmax_scale, window)
    stream = torch.cuda.current_stream().cuda_stream
    _lib.check(lib.sink_attn_bwd_noalloc(ctypes.byref(p), q.data_ptr(), k.data_ptr(), d["v"].data_ptr(),
                                         d["sinks"].data_ptr(), d["o"].data_ptr(), d["lse"].data_ptr(),
                                         d["dout"].data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                         ds.data_ptr(), stream))
    return dq, dk, dv, ds


def _case(w, window, seed):
    import attention_sink_fwd_amd as sa

    d = {n: t.to("cuda:0") for n, t in make_inputs(w, seed=seed).items()}
    d["o"], d["lse"] = sa.sink_attn_fwd(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens"], w.max_seqlen,
                                        w.softmax_scale, window)
    ref = sa.sink_attn_bwd(d["q"], d["k"], d["v"], d["sinks"], d["o"], d["lse"], d["dout"], d["cu_seqlens"],
                           w.max_seqlen, w.softmax_scale, window)
    got = _call_noalloc(d, w, window)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_backward_matches_workspace_backward_twice():
    big = WORKLOADS[2]
    small = custom_workload((300, 5, 190), 8, 2, 64, 37, "bf16")
    for w, window, seed, same_split in ((big, 0, 2, False), (small, 37, 11, True)):
        say("case no-alloc backward", w.name, w.lengths[:4], "window", window)
        ref, got = _case(w, window, seed)
        assert torch.equal(got[0], ref[0]), "dq"
        assert torch.equal(got[3], ref[3]), "dsinks"
        for name, a, b in (("dk", got[1], ref[1]), ("dv", got[2], ref[2])):
            if same_split:
                assert torch.equal(a, b), name
            e = rel_l2(f64(a), f64(b))
            say(f"  {name}: rel-L2 against sink_attn_bwd {e:.2e}")
            assert e <= TOL_GRAD, name
        assert rel_l2(f64(got[3]), f64(ref[3])) <= TOL_DS
        for t in got:
            assert torch.isfinite(t).all()


def _noalloc_into(d, w, window, outs, stream):
    import attention_sink_fwd_amd as sa

    lib = _lib.load()
    q, k = d["q"], d["k"]
    dq, dk, dv, ds = outs
    p = sa.make_params(q, k, d["cu_seqlens"], w.max_seqlen, w.softmax_scale, window)
    _lib.check(lib.sink_attn_bwd_noalloc(ctypes.byref(p), q.data_ptr(), k.data_ptr(), d["v"].data_ptr(),
                                         d["sinks"].data_ptr(), d["o"].data_ptr(), d["lse"].data_ptr(),
                                         d["dout"].data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                         ds.data_ptr(), stream.cuda_stream))


@pytest.mark.parametrize("window", [0, 96])
def test_noalloc_backward_replays_in_a_hip_graph(window):
    """Captured in a HIP graph -- the use the entry point is for -- and
    replayed three times, with eager work and a synchronisation between the
    replays: every replay gives the eager call's bits (window 96 runs the
    fused short-window kernel)."""
    import attention_sink_fwd_amd as sa

    w = custom_workload((300, 5, 190), 8, 2, 64, window, "bf16")
    say("case no-alloc backward in a graph, window", window)
    d = {n: t.to("cuda:0") for n, t in make_inputs(w, seed=23 + window).items()}
    d["o"], d["lse"] = sa.sink_attn_fwd(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens"], w.max_seqlen,
                                        w.softmax_scale, window)
    ref = [torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["k"]), torch.empty_like(d["sinks"])]
    _noalloc_into(d, w, window, ref, torch.cuda.current_stream())
    torch.cuda.synchronize()
    outs = [torch.empty_like(t) for t in ref]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _noalloc_into(d, w, window, outs, side)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        _noalloc_into(d, w, window, outs, torch.cuda.current_stream())
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "dsinks"), outs, ref):
            assert torch.equal(a, b), (rep, name)
