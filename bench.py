#!/usr/bin/env python3
"""Sink-attention forward + backward throughput on one MI355X.

One step = the whole hot path on one batch of synthetic input already
resident in HBM: host dispatch, the forward kernel (O, LSE), then the
backward (dQ kernel with the row statistics D_i, dK/dV kernel, epilogue
with dS_h).
Default workload: GPT-OSS-20B-shaped attention, B=1, Hq=64, Hkv=8, d=64,
L=4096, causal, bf16.

Prints ONE JSON line.  Throughput counts algorithmic flops (14*d per visible
query/key pair per query head: 4d forward, 10d backward).  Untimed passes
first time each kernel alone, bracketed by two HIP events per step
(kernel_ms), and pick the dominant (longest) matrix-core kernel; in the
timed region only that kernel is bracketed, the same way, on the stream it
runs on, and the roofline object reports it.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sink-attn fwd+bwd TFLOP/s + % bf16 MFMA peak, Hq64/Hkv8/d64 L=4096 causal"
PEAK_BF16_TFLOPS = 2500.0  # MI355X published dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


class Hip:
    """The few HIP runtime calls the timing needs (same runtime torch uses)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        vp = ctypes.c_void_p
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [vp, vp]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        self.lib.hipEventDestroy.argtypes = [vp]

    # Timing-only events: without a system-scope release (hipEventDisableSystemFence),
    # recording one does not write back and invalidate L2 between the kernels
    # it separates; the host reads them only after a device synchronisation.
    DISABLE_SYSTEM_FENCE = 0x20000000

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) == 0
        return e

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, stream) == 0

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return float(out.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


def sources_sha256(paths):
    """sha256 over the concatenated bytes of the given repo files, in order."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_for_current_kernel(kernel, workload):
    """HBM bytes per launch of `kernel` from rocprofv3 FETCH_SIZE + WRITE_SIZE.

    Taken from profiles/traffic.json, and only for the workload the counters
    were measured on, while the kernel's sources are byte-identical to the
    ones they were measured on; else None.
    """
    try:
        with open(TRAFFIC_FILE) as f:
            entry = json.load(f)[f"{kernel}@{workload}"]
        if entry.get("workload") != workload:
            return None
        if entry.get("sources_sha256") != sources_sha256(entry["sources"]):
            return None
        return float(entry["bytes_per_launch"])
    except (OSError, ValueError, KeyError, TypeError):
        return None


def cpu_baseline(inp, w, min_seconds=10.0):
    """The oracle (unchanged), timed on the host over whole KV groups of the
    same workload: group after group until at least ``min_seconds`` passed."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = None
    grp = w.num_q_heads // w.num_kv_heads
    done = 0
    t0 = time.perf_counter()
    while done < w.num_kv_heads and (time.perf_counter() - t0) < min_seconds:
        g = done
        oracle.forward(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["cu_seqlens"],
                       w.softmax_scale, w.window, heads=list(range(g * grp, (g + 1) * grp)))
        oracle.backward(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["dout"],
                        inp["cu_seqlens"], w.softmax_scale, w.window, kv_heads=[g])
        done += 1
    dt = time.perf_counter() - t0
    flops = w.flops()["total"] * done / w.num_kv_heads
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads if threads is not None else os.cpu_count(),
        "kind": "oracle",
        "sample": (f"KV groups 0-{done - 1} (query heads 0-{done * grp - 1}) of {w.name}: "
                   f"float64 forward + backward, {flops / 1e9:.1f} GFLOP in {dt:.1f} s"),
    }


def calibrate_copy(nbytes=1 << 30):
    """A plain copy kernel of known size for scaling rocprofv3's FETCH_SIZE /
    WRITE_SIZE: torch.neg over float32 reads and writes nbytes each."""
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "torch.neg float32", "bytes_read_per_launch": nbytes,
                      "bytes_written_per_launch": nbytes, "launches": 3}), flush=True)


def paged_decode(args):
    """One decode step over a paged KV cache: 64 sequences with 4096 cached
    keys each (64-key pages in a seeded random order), one new token per
    sequence, GPT-OSS attention shape.  Reports the rate at which the step
    reads the cache (each sequence's keys and values once per KV head)
    against the HBM peak.  Inputs are synthetic (seeded normal values)."""
    import torch

    import attention_sink_fwd_amd as sa

    nseq, ctx, hq, hkv, d, ps = 64, 4096, 64, 8, 64, 64
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    pages = nseq * ctx // ps
    k_cache = torch.randn((pages, ps, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
    v_cache = torch.randn((pages, ps, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
    perm = torch.randperm(pages, generator=gen, device=dev).to(torch.int32)
    block_table = perm.view(nseq, ctx // ps).contiguous()
    kv_lens = torch.full((nseq,), ctx, dtype=torch.int32, device=dev)
    q = torch.randn((nseq, hq, d), generator=gen, device=dev).to(torch.bfloat16)
    sinks = torch.randn((hq,), generator=gen, device=dev)
    cu = torch.arange(nseq + 1, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((hq, nseq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    hip = Hip()

    def step():
        sa.sink_attn_fwd_paged(q, k_cache, v_cache, block_table, kv_lens, sinks, cu, 1, None, 0,
                               o=o, lse=lse, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    evs = [(hip.event(), hip.event()) for _ in range(K)]
    t0 = time.perf_counter()
    for a, b in evs:
        hip.record(a, sh)
        step()
        hip.record(b, sh)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_ms = sum(hip.ms(a, b) for a, b in evs) / K
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    kv_bytes = 2.0 * nseq * ctx * hkv * d * 2  # K and V, bf16, read once per KV head
    io_bytes = 2.0 * nseq * hq * d * 2 + nseq * hq * 4 + kv_bytes
    ms = (t1 - t0) * 1000.0 / K
    gbs = io_bytes / (kern_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "sink-attn paged decode step, KV-cache read GB/s (64 seqs x 4096 ctx, Hq64/Hkv8/d64)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "paged_decode_b64_ctx4096_hq64_hkv8_d64_page64", "num_seqs": nseq,
                   "context": ctx, "page_size": ps, "new_tokens_per_seq": 1},
        "tokens_per_s": round(nseq / (kern_ms * 1e-3), 1),
        "roofline": {"kernel": "fwd_paged", "kernel_ms": round(kern_ms, 5), "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": io_bytes,
                     "traffic": traffic_for_current_kernel(
                         "fwd_paged", "paged_decode_b64_ctx4096_hq64_hkv8_d64_page64")},
    }), flush=True)


def token_logps(args):
    """One step of per-token log-probabilities and their gradient: 8192
    positions over GPT-OSS's 201,088-entry vocabulary in bfloat16 (3.3 GB of
    logits), seeded normal logits.  Each kernel is bracketed with HIP events
    on its stream; the rate counts the bytes each kernel must move (logits
    read once by each, the gradient written once, the per-row vectors)."""
    import torch

    import attention_sink_fwd_amd as sa
    from synthetic.workloads import make_logits_device

    rows, vocab = 8192, 201088
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = make_logits_device(rows, vocab, "bf16", seed=1234, device="cuda:0")
    x, ids, g = d["logits"], d["ids"], d["grad"]
    logps = torch.empty((rows,), dtype=torch.float32, device=dev)
    lse = torch.empty_like(logps)
    gx = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    lib = sa._lib.load()
    hip = Hip()

    def step(ev=None):
        if ev:
            hip.record(ev[0], sh)
        sa._lib.check(lib.token_logps_fwd(x.data_ptr(), 0, 1, rows, vocab, 0, vocab, ids.data_ptr(),
                                          logps.data_ptr(), lse.data_ptr(), sh))
        if ev:
            hip.record(ev[1], sh)
        sa._lib.check(lib.token_logps_bwd(x.data_ptr(), 0, 1, rows, vocab, 0, vocab, ids.data_ptr(),
                                          lse.data_ptr(), g.data_ptr(), gx.data_ptr(), 0, vocab, sh))
        if ev:
            hip.record(ev[2], sh)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    evs = [(hip.event(), hip.event(), hip.event()) for _ in range(K)]
    t0 = time.perf_counter()
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    fwd_ms = sum(hip.ms(a, b) for a, b, _ in evs) / K
    bwd_ms = sum(hip.ms(b, c) for _, b, c in evs) / K
    for ev in evs:
        for e in ev:
            hip.destroy(e)
    xb = float(rows) * vocab * 2
    fwd_bytes = xb + rows * (4 + 4 + 4)          # logits, ids in; logp, lse out
    bwd_bytes = 2 * xb + rows * (4 + 4 + 4)      # logits in, grad out; ids, lse, g in
    step_gbs = (fwd_bytes + bwd_bytes) / ((fwd_ms + bwd_ms) * 1e-3) / 1e9
    dom, dom_ms, dom_bytes = ("logps_bwd", bwd_ms, bwd_bytes) if bwd_ms >= fwd_ms else \
        ("logps_fwd", fwd_ms, fwd_bytes)
    ach = dom_bytes / (dom_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "per-token log-prob fwd+bwd, HBM GB/s (8192 positions x 201088 vocab, bf16)",
        "value": round(step_gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1000.0 / K, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "token_logps_rows8192_vocab201088", "rows": rows, "vocab": vocab},
        "kernel_ms": {"logps_fwd": round(fwd_ms, 5), "logps_bwd": round(bwd_ms, 5)},
        "roofline": {"kernel": dom, "kernel_ms": round(dom_ms, 5), "bound": "hbm",
                     "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(ach / PEAK_HBM_GBS, 4), "algorithmic_bytes": dom_bytes,
                     "traffic": traffic_for_current_kernel(dom, "token_logps_rows8192_vocab201088")},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, help="workload id 1-5 (default 2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--paged-decode", action="store_true",
                    help="time one decode step over a paged KV cache instead (own JSON line)")
    ap.add_argument("--token-logps", action="store_true",
                    help="time the per-token log-probability kernels instead")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a known-size copy kernel (for rocprofv3 counter scaling)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: --gpus {args.gpus} (WORLD_SIZE={world}) requested, but this build runs "
              "on one GPU only: the kernel works on one GPU's head share and there is no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.token_logps:
        token_logps(args)
        return
    if args.paged_decode:
        paged_decode(args)
        return

    import torch

    import attention_sink_fwd_amd as sa
    from attention_sink_fwd_amd import _lib
    from synthetic.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(w)
    d = {k: v.to(dev) for k, v in inp.items()}
    q, k, v, s, cu, do = d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens"], d["dout"]
    o = torch.empty_like(q)
    lse = torch.empty((w.num_q_heads, w.total_tokens), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ds = torch.empty_like(s)
    ws_bytes = sa.sink_attn_bwd_workspace_size(q, k, cu, w.max_seqlen, w.softmax_scale, w.window)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    lib = _lib.load()
    hip = Hip()

    def step():
        sa.sink_attn_fwd(q, k, v, s, cu, w.max_seqlen, w.softmax_scale, w.window, o=o, lse=lse,
                         stream=stream)
        sa.sink_attn_bwd(q, k, v, s, o, lse, do, cu, w.max_seqlen, w.softmax_scale, w.window,
                         dq=dq, dk=dk, dv=dv, dsinks=ds, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    sh = ctypes.c_void_p(stream.cuda_stream)

    def run_steps(n, fwd_events, bwd_events):
        """n steps; fwd_events(i) -> (start, end) or None, bwd_events(i) -> 4 handles."""
        for i in range(n):
            fe = fwd_events(i)
            if fe:
                hip.record(fe[0], sh)
            sa.sink_attn_fwd(q, k, v, s, cu, w.max_seqlen, w.softmax_scale, w.window, o=o,
                             lse=lse, stream=stream)
            if fe:
                hip.record(fe[1], sh)
            arr = (ctypes.c_void_p * 4)(*bwd_events(i))
            _lib.check(lib.sink_attn_set_bwd_events(arr))
            sa.sink_attn_bwd(q, k, v, s, o, lse, do, cu, w.max_seqlen, w.softmax_scale, w.window,
                             dq=dq, dk=dk, dv=dv, dsinks=ds, workspace=ws, stream=stream)
        _lib.check(lib.sink_attn_set_bwd_events(None))

    # Untimed passes, one per kernel, each bracketing only that kernel with
    # two events per step (as the timed region brackets the dominant one):
    # the per-kernel breakdown and the dominant kernel.  (Bracketing every
    # kernel in one pass would add an event packet between each pair of
    # kernels and inflate each kernel's time.)
    nb = min(args.steps, 20)

    def avg(evs, a, b):
        return sum(hip.ms(e[a], e[b]) for e in evs) / len(evs)

    # Short windows run one fused backward kernel in place of the dQ and dK/dV
    # kernels (its launch fills the first event slot pair).
    fused = sa.sink_attn_bwd_fused(q, k, cu, w.max_seqlen, w.softmax_scale, w.window)
    bwd_kernels = ("bwd_fused",) if fused else ("bwd_dq", "bwd_dkdv")
    slot = {"bwd_dq": 0, "bwd_fused": 0, "bwd_dkdv": 1, "bwd_post": 2}
    kernel_ms = {}
    for kname in ("fwd", *bwd_kernels, "bwd_post"):
        evb = [[hip.event() for _ in range(2)] for _ in range(nb)]
        if kname == "fwd":
            fe, be = (lambda i: (evb[i][0], evb[i][1])), (lambda i: (None, None, None, None))
        else:
            j = slot[kname]

            def be(i, j=j):
                h = [None, None, None, None]
                h[j], h[j + 1] = evb[i][0].value, evb[i][1].value
                return tuple(h)
            fe = lambda i: None  # noqa: E731
        run_steps(nb, fe, be)
        torch.cuda.synchronize()
        kernel_ms[kname] = avg(evb, 0, 1)
        for row in evb:
            for e in row:
                hip.destroy(e)
    kms = {kname: kernel_ms[kname] for kname in ("fwd", *bwd_kernels)}
    dom = max(kms, key=kms.get)

    # Timed region: K steps; only the dominant kernel is bracketed (two
    # events per step on the stream it runs on).
    K = args.steps
    evt = [[hip.event() for _ in range(2)] for _ in range(K)]
    none = None
    if dom == "fwd":
        fwd_ev, bwd_ev = (lambda i: (evt[i][0], evt[i][1])), (lambda i: (none, none, none, none))
    elif slot[dom] == 0:
        fwd_ev, bwd_ev = (lambda i: None), (lambda i: (evt[i][0].value, evt[i][1].value, none, none))
    else:
        fwd_ev, bwd_ev = (lambda i: None), (lambda i: (none, evt[i][0].value, evt[i][1].value, none))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(K, fwd_ev, bwd_ev)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dom_ms = avg(evt, 0, 1)
    for row in evt:
        for e in row:
            hip.destroy(e)

    ms = (t1 - t0) * 1000.0 / K
    fl = w.flops()
    tflops = fl["total"] / (ms * 1e-3) / 1e12
    # Algorithmic flops per launch of each matrix-core kernel (FA convention,
    # 2*d flops per visible pair per product): forward 2 products (S, PV);
    # dK/dV kernel 4 of the 5 backward products (S, dP, dV, dK); dQ kernel the
    # remaining one (dQ) -- its recomputed S and dP are not counted; the fused
    # short-window kernel all 5.
    pairs = w.visible_pairs()
    algo = {"fwd": 4.0 * w.head_dim * pairs, "bwd_dkdv": 8.0 * w.head_dim * pairs,
            "bwd_dq": 2.0 * w.head_dim * pairs, "bwd_fused": 10.0 * w.head_dim * pairs}
    # Matrix work each kernel executes on visible pairs: the dQ kernel
    # recomputes S and dP (2 more products per pair than it is credited with).
    executed = dict(algo, bwd_dq=6.0 * w.head_dim * pairs)

    def frac(kname, flops):
        return round(flops / (kms[kname] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    kernel_frac = {"fwd": frac("fwd", algo["fwd"])}
    if fused:
        kernel_frac["bwd_fused"] = frac("bwd_fused", algo["bwd_fused"])
    else:
        kernel_frac["bwd_dq"] = {"credited": frac("bwd_dq", algo["bwd_dq"]),
                                 "executed": frac("bwd_dq", executed["bwd_dq"])}
        kernel_frac["bwd_dkdv"] = frac("bwd_dkdv", algo["bwd_dkdv"])
    dom_tflops = algo[dom] / (dom_ms * 1e-3) / 1e12
    traffic = traffic_for_current_kernel(dom, w.name)
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": len(w.lengths),
            "seq_len": w.max_seqlen,
            "total_tokens": w.total_tokens,
            "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "window": w.window,
            "causal": True,
            "flops_per_step": fl["total"],
        },
        "pct_bf16_mfma_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "kernel_ms": {kname: round(val, 4) for kname, val in kernel_ms.items()},
        "kernel_ms_note": ("each kernel timed in its own untimed pass, bracketed alone by two events per "
                           "step; sum minus ms_per_step: event overhead and launch gaps"),
        "kernel_sum_minus_step_ms": round(sum(kernel_ms.values()) - ms, 4),
        "kernel_tflops": {kname: round(algo[kname] / (kms[kname] * 1e-3) / 1e12, 1) for kname in kms},
        "kernel_frac": kernel_frac,
        "roofline": {
            "kernel": dom,
            "kernel_ms": round(dom_ms, 4),
            "bound": "mfma",
            "achieved": round(dom_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(dom_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
