"""Per-token log-probabilities, written out from their definition in
float64 on the CPU.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test
suite, the smoke check and the benchmark's CPU-baseline leg may use it; the
HIP path shares no code with it.

Source: the MiniMind tutorial page "强化学习:GRPO 与 PPO", Part 7 "Rollout
引擎", subsection "LogProb 计算": the log-probability of each sampled token
is its entry of log_softmax(logits) over the vocabulary, taken at the
token's id.  Written out for row i of logits x (one token position):

    lse_i  = ln sum_v exp(x_iv)
    logp_i = x_i,id_i - lse_i
    d logp_i / d x_iv = [v == id_i] - exp(x_iv - lse_i)

so an upstream gradient g_i gives dL/dx_iv = g_i ([v == id_i] - softmax_iv).
Library primitive used as a step: ``scipy.special.logsumexp``.
"""
from __future__ import annotations

import numpy as np
from scipy.special import logsumexp


def _f64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def token_logps(logits, ids):
    """(logp [N], lse [N]) in float64 for logits [N, V] and ids [N]; an id
    outside [0, V) gives logp = NaN."""
    x = _f64(logits)
    ids = np.asarray(_f64(ids), dtype=np.int64)
    lse = logsumexp(x, axis=1)
    ok = (ids >= 0) & (ids < x.shape[1])
    picked = np.where(ok, x[np.arange(x.shape[0]), np.clip(ids, 0, x.shape[1] - 1)], np.nan)
    return picked - lse, lse


def token_logps_grad(logits, ids, grad_logps):
    """dL/dlogits [N, V] (float64) for upstream dL/dlogp = grad_logps [N]."""
    x = _f64(logits)
    ids = np.asarray(_f64(ids), dtype=np.int64)
    g = _f64(grad_logps)
    _, lse = token_logps(x, ids)
    out = -g[:, None] * np.exp(x - lse[:, None])
    ok = (ids >= 0) & (ids < x.shape[1])
    rows = np.arange(x.shape[0])[ok]
    out[rows, ids[ok]] += g[ok]
    return out
