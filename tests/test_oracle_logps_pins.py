"""Pins of the per-token log-probability oracle (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
from synthetic.workloads import make_logits


def test_matches_torch_log_softmax_and_gather():
    d = make_logits(37, 1003, "f32", seed=1)
    x = d["logits"].double()
    ref = torch.log_softmax(x, dim=1).gather(1, d["ids"].long()[:, None])[:, 0]
    logp, lse = oracle.token_logps(d["logits"], d["ids"])
    assert np.abs(logp - ref.numpy()).max() < 1e-12
    assert np.abs(lse - torch.logsumexp(x, dim=1).numpy()).max() < 1e-12


def test_gradient_matches_torch_autograd():
    d = make_logits(11, 257, "f32", seed=2)
    x = d["logits"].double().requires_grad_(True)
    lp = torch.log_softmax(x, dim=1).gather(1, d["ids"].long()[:, None])[:, 0]
    (lp * d["grad"].double()).sum().backward()
    got = oracle.token_logps_grad(d["logits"], d["ids"], d["grad"])
    assert np.abs(got - x.grad.numpy()).max() < 1e-12


def test_closed_forms_and_invariants():
    V = 500
    x = np.full((3, V), 2.5)
    logp, lse = oracle.token_logps(x, np.array([0, 7, V - 1]))
    assert np.allclose(logp, -math.log(V), atol=1e-13)
    assert np.allclose(lse, 2.5 + math.log(V), atol=1e-13)
    d = make_logits(5, 300, "f32", seed=3)
    a, _ = oracle.token_logps(d["logits"], d["ids"])
    shift = torch.arange(5, dtype=torch.float64)[:, None] * 7.0
    b, _ = oracle.token_logps(d["logits"].double() + shift, d["ids"])
    assert np.abs(a - b).max() < 1e-9
    g = oracle.token_logps_grad(d["logits"], d["ids"], d["grad"])
    assert np.abs(g.sum(axis=1)).max() < 1e-12  # softmax rows sum to one
    # one dominant logit: its log-probability tends to 0
    y = np.zeros((1, 50))
    y[0, 9] = 60.0
    assert abs(oracle.token_logps(y, np.array([9]))[0][0]) < 1e-20


def test_out_of_range_ids_give_nan_and_no_gather_term():
    d = make_logits(3, 40, "f32", seed=4)
    ids = torch.tensor([-1, 5, 40], dtype=torch.int32)
    logp, _ = oracle.token_logps(d["logits"], ids)
    assert np.isnan(logp[0]) and np.isnan(logp[2]) and np.isfinite(logp[1])
    g = oracle.token_logps_grad(d["logits"], ids, torch.ones(3))
    assert np.all(g[0] < 0) and np.all(g[2] < 0)


def test_finite_differences():
    d = make_logits(2, 9, "f32", seed=5)
    x = d["logits"].double().numpy()
    ids = d["ids"].numpy()
    g = d["grad"].double().numpy()
    got = oracle.token_logps_grad(x, ids, g)
    h = 1e-6
    for i in range(2):
        for v in range(9):
            xp, xm = x.copy(), x.copy()
            xp[i, v] += h
            xm[i, v] -= h
            fd = (np.dot(oracle.token_logps(xp, ids)[0], g) - np.dot(oracle.token_logps(xm, ids)[0], g)) / (2 * h)
            assert abs(fd - got[i, v]) < 1e-7


@pytest.mark.parametrize("mistake", ["sign", "no_shift", "wrong_row"])
def test_planted_mistakes_are_caught(mistake):
    """A plausible slip in the definition fails the library pin."""
    d = make_logits(6, 64, "f32", seed=6)
    x = d["logits"].double().numpy()
    ids = d["ids"].numpy().astype(np.int64)
    lse = np.log(np.exp(x).sum(axis=1))
    if mistake == "sign":
        bad = lse - x[np.arange(6), ids]
    elif mistake == "no_shift":
        bad = x[np.arange(6), ids]
    else:
        bad = x[np.arange(6), ids[::-1]] - lse
    ref = torch.log_softmax(torch.from_numpy(x), 1).gather(1, torch.from_numpy(ids)[:, None])[:, 0].numpy()
    assert np.abs(bad - ref).max() > 1e-3
