"""Helpers for the GPU-vs-oracle parity tests.

Tolerances (float results of the bf16 matrix-core path against the float64
oracle on identical inputs):
  O, LSE        max |gpu - ref| <= 2e-2 over the compared elements
  dQ, dK, dV    ||gpu - ref||_2 / ||ref||_2 <= 2e-2 over the compared tensor
  dS            ||gpu - ref||_2 / ||ref||_2 <= 1e-2 over the [Hq] vector
A reference norm below 1e-6 (a sink of +30 drives everything to ~0) switches
the relative checks to the same bound on the absolute norm.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import torch

TOL_O = 2e-2
TOL_LSE = 2e-2
TOL_GRAD = 2e-2
TOL_DS = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a, ref):
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(a - ref)
    return num / den if den > 1e-6 else num


def max_abs(a, ref):
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - ref)))


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def run_gpu(inputs, max_seqlen, scale, window, device="cuda:0"):
    """Forward + backward through the C ABI; returns float64 numpy results."""
    import attention_sink_fwd_amd as sa

    d = {k: v.to(device) for k, v in inputs.items()}
    o, lse = sa.sink_attn_fwd(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens"], max_seqlen,
                              scale, window)
    dq, dk, dv, ds = sa.sink_attn_bwd(d["q"], d["k"], d["v"], d["sinks"], o, lse, d["dout"],
                                      d["cu_seqlens"], max_seqlen, scale, window)
    torch.cuda.synchronize()
    out = {"o": f64(o), "lse": f64(lse), "dq": f64(dq), "dk": f64(dk), "dv": f64(dv),
           "ds": f64(ds)}
    for name, arr in out.items():
        assert np.all(np.isfinite(arr)), f"non-finite values in GPU {name}"
    return out


def check_full(gpu, ref, label=""):
    """Compare every element of a full oracle result."""
    errs = {
        "o": max_abs(gpu["o"], ref["o"]),
        "lse": max_abs(gpu["lse"], ref["lse"]),
        "dq": rel_l2(gpu["dq"], ref["dq"]),
        "dk": rel_l2(gpu["dk"], ref["dk"]),
        "dv": rel_l2(gpu["dv"], ref["dv"]),
        "ds": rel_l2(gpu["ds"], ref["ds"]),
    }
    say(f"  {label} errors: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert errs["o"] <= TOL_O, (label, errs)
    assert errs["lse"] <= TOL_LSE, (label, errs)
    assert errs["dq"] <= TOL_GRAD and errs["dk"] <= TOL_GRAD and errs["dv"] <= TOL_GRAD, (label, errs)
    assert errs["ds"] <= TOL_DS, (label, errs)
    return errs


def record_errors(config: str, compared: str, errs: dict) -> None:
    """Append one line of error figures to the file named by
    SINK_ATTN_ERROR_LOG (when set): the per-workload error report."""
    path = os.environ.get("SINK_ATTN_ERROR_LOG")
    if not path:
        return
    row = {"config": config, "compared": compared}
    row.update({k: float(v) for k, v in errs.items()})
    with open(path, "a") as f:
        f.write(json.dumps(row) + "\n")
