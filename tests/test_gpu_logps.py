"""Per-token log-probability kernels on the GPU, through the C ABI.

Compared element by element with the float64 oracle (``oracle.token_logps``,
``oracle.token_logps_grad``) on the same seeded logits.  Tolerances, from the
arithmetic (float32 accumulation of exp over the row in a fixed tree, one
rounding of the gradient to the logits' type):
  logp, lse   |gpu - ref| <= 1e-4 + 2e-6 |ref|
  grad        |gpu - ref| <= rtol |g| (p + [v == id]) + 1e-30,
              rtol = 2^-8 for bfloat16 output, 1e-4 for float32
where p = exp(x - lse) is the oracle's softmax entry and g the upstream
gradient of the row (the bound is relative to the size of the terms, so it
stays meaningful where g (delta - p) cancels).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synthetic.workloads import make_logits, make_logits_device
from tests.parity_util import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
RTOL_GRAD = {"bf16": 2.0 ** -8, "f32": 1e-4}

CASES = [
    # rows, vocab, dtype, row stride (None: contiguous)
    (64, 1024, "bf16", None),
    (33, 1003, "bf16", 1008),       # ragged tail of 3
    (17, 7, "f32", 8),              # shorter than one chunk
    (5, 1, "bf16", 8),              # a one-token vocabulary
    (40, 32773, "f32", 32776),      # whole unrolled passes and a tail of 5
    (9, 50000, "bf16", 50048),      # unrolled passes plus single chunks
    (3, 6400, "bf16", None),
]


def _to_dev(d, stride=None):
    x = d["logits"]
    if stride is not None and x.stride(0) != stride:
        buf = torch.full((x.shape[0], stride), float("nan"), dtype=x.dtype)
        buf[:, : x.shape[1]] = x
        x = buf[:, : x.shape[1]]
    dev = torch.empty_strided(x.shape, x.stride(), dtype=x.dtype, device=DEV)
    dev.copy_(x)
    return dev, d["ids"].to(DEV), d["grad"].to(DEV)


def _check_fwd(logp, lse, x_cpu, ids_cpu, label):
    ref_lp, ref_lse = oracle.token_logps(x_cpu, ids_cpu)
    lp = logp.cpu().double().numpy()
    ls = lse.cpu().double().numpy()
    assert np.array_equal(np.isnan(lp), np.isnan(ref_lp)), label
    ok = ~np.isnan(ref_lp)
    e_lp = np.abs(lp[ok] - ref_lp[ok]) - 2e-6 * np.abs(ref_lp[ok])
    e_ls = np.abs(ls - ref_lse) - 2e-6 * np.abs(ref_lse)
    say(f"{label}: logp err {np.max(np.abs(lp[ok] - ref_lp[ok]), initial=0):.2e} "
        f"lse err {np.max(np.abs(ls - ref_lse), initial=0):.2e}")
    assert np.max(e_lp, initial=0) <= 1e-4, label
    assert np.max(e_ls, initial=0) <= 1e-4, label
    return ref_lse


def _check_grad(gx, x_cpu, ids_cpu, g_cpu, dtype, label):
    ref = oracle.token_logps_grad(x_cpu, ids_cpu, g_cpu)
    got = gx.cpu().double().numpy()
    x = x_cpu.double().numpy()
    _, lse = oracle.token_logps(x_cpu, ids_cpu)
    p = np.exp(x - lse[:, None])
    ids = ids_cpu.numpy().astype(np.int64)
    delta = np.zeros_like(p)
    ok = (ids >= 0) & (ids < x.shape[1])
    delta[np.arange(x.shape[0])[ok], ids[ok]] = 1.0
    bound = RTOL_GRAD[dtype] * np.abs(g_cpu.double().numpy())[:, None] * (p + delta) + 1e-30
    err = np.abs(got - ref)
    say(f"{label}: grad max err {err.max(initial=0):.2e}, worst err/bound {np.max(err / bound, initial=0):.3f}")
    assert np.all(err <= bound), label


@pytest.mark.parametrize("rows,vocab,dtype,stride", CASES)
def test_matches_oracle(rows, vocab, dtype, stride):
    import attention_sink_fwd_amd as sa

    label = f"logps rows={rows} V={vocab} {dtype} stride={stride}"
    say(label)
    d = make_logits(rows, vocab, dtype, seed=rows * 7 + vocab)
    x, ids, g = _to_dev(d, stride)
    logp, lse = sa.token_logps_fwd(x, ids)
    gx = sa.token_logps_bwd(x, ids, lse, g)
    torch.cuda.synchronize()
    _check_fwd(logp, lse, d["logits"], d["ids"], label)
    _check_grad(gx, d["logits"], d["ids"], d["grad"], dtype, label)
    if vocab == 1:
        assert torch.all(logp == 0)


def test_bad_ids_give_nan_and_no_gather_term():
    import attention_sink_fwd_amd as sa

    d = make_logits(6, 300, "bf16", seed=11, row_stride=304)
    d["ids"] = torch.tensor([-1, 0, 299, 300, 2 ** 31 - 1, -(2 ** 31)], dtype=torch.int32)
    x, ids, g = _to_dev(d, 304)
    logp, lse = sa.token_logps_fwd(x, ids)
    gx = sa.token_logps_bwd(x, ids, lse, g)
    torch.cuda.synchronize()
    lp = logp.cpu()
    assert torch.isnan(lp[[0, 3, 4, 5]]).all() and torch.isfinite(lp[[1, 2]]).all()
    _check_fwd(logp, lse, d["logits"], d["ids"], "bad ids")
    _check_grad(gx, d["logits"], d["ids"], d["grad"], "bf16", "bad ids")


def test_masked_vocabulary_entries():
    """-inf logits (a masked or padded part of the vocabulary) contribute nothing."""
    import attention_sink_fwd_amd as sa

    d = make_logits(4, 2051, "f32", seed=12, row_stride=2056)
    x = d["logits"].clone()
    x[0, 1000:] = -math.inf        # long masked run, across chunks and the tail
    x[1, ::3] = -math.inf          # scattered
    x[2, :] = -math.inf
    x[2, 1234] = 5.0               # only one token possible: logp 0 there
    x[3, :2048] = -math.inf        # only the ragged tail left
    ids = torch.tensor([5, 1, 1234, 2049], dtype=torch.int32)
    d.update(logits=x, ids=ids)
    xd, idd, g = _to_dev(d, 2056)
    logp, lse = sa.token_logps_fwd(xd, idd)
    gx = sa.token_logps_bwd(xd, idd, lse, g)
    torch.cuda.synchronize()
    _check_fwd(logp, lse, x, ids, "masked")
    assert logp[2].item() == 0.0
    _check_grad(gx, x, ids, d["grad"], "f32", "masked")


def test_padding_columns_of_the_gradient_are_not_written():
    import attention_sink_fwd_amd as sa

    d = make_logits(8, 1001, "bf16", seed=13, row_stride=1008)
    x, ids, g = _to_dev(d, 1008)
    _, lse = sa.token_logps_fwd(x, ids)
    buf = torch.full((8, 1016), 7.0, dtype=torch.bfloat16, device=DEV)
    gx = sa.token_logps_bwd(x, ids, lse, g, grad_logits=buf[:, :1001])
    torch.cuda.synchronize()
    assert torch.all(buf[:, 1001:] == 7.0)
    _check_grad(gx, d["logits"], d["ids"], d["grad"], "bf16", "padded grad")


def test_bitwise_reproducible_and_autograd_matches_entry_points():
    import attention_sink_fwd_amd as sa

    d = make_logits(128, 20000, "bf16", seed=14)
    x, ids, g = _to_dev(d)
    a = sa.token_logps_fwd(x, ids)
    b = sa.token_logps_fwd(x, ids)
    ga = sa.token_logps_bwd(x, ids, a[1], g)
    gb = sa.token_logps_bwd(x, ids, b[1], g)
    xr = x.clone().requires_grad_(True)
    lp = sa.token_logps(xr, ids)
    lp.backward(g)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(ga, gb)
    assert torch.equal(lp.detach(), a[0])
    assert torch.equal(xr.grad, ga)


@pytest.mark.parametrize("position_major", [False, True])
def test_strided_batch_view_is_read_in_place(position_major):
    """The rollout layout: logits [B, T + 1, V] from the model, log-probs of
    logits[:, :-1, :] against input_ids[:, 1:] (no copy of the logits); also
    a [T + 1, B, V] buffer viewed as [B, T + 1, V]."""
    import attention_sink_fwd_amd as sa

    B, T, V = 3, 37, 1000
    d = make_logits(B * (T + 1), V, "bf16", seed=16)
    full = d["logits"].view(B, T + 1, V)
    if position_major:
        full = full.view(T + 1, B, V).transpose(0, 1)     # strides (V, B*V, 1)
    gen = np.random.default_rng(17)
    input_ids = torch.from_numpy(gen.integers(0, V, size=(B, T + 1)).astype(np.int32))
    g = d["grad"][: B * T].view(B, T)
    dev_full = torch.empty_strided(full.shape, full.stride(), dtype=full.dtype, device=DEV)
    dev_full.copy_(full)
    xs = dev_full[:, :-1, :]
    ids = input_ids[:, 1:].to(DEV)                          # a strided view; the binding packs it
    logp, lse = sa.token_logps_fwd(xs, ids)
    gx = sa.token_logps_bwd(xs, ids, lse, g.to(DEV))
    torch.cuda.synchronize()
    assert logp.shape == (B, T) and gx.shape == (B, T, V) and gx.stride() == xs.stride()
    x_cpu = full[:, :-1, :].reshape(B * T, V)
    ids_cpu = input_ids[:, 1:].reshape(-1)
    label = f"strided view position_major={position_major}"
    _check_fwd(logp.reshape(-1), lse.reshape(-1), x_cpu, ids_cpu, label)
    _check_grad(gx.reshape(B * T, V), x_cpu, ids_cpu, g.reshape(-1), "bf16", label)


def test_zero_rows():
    import attention_sink_fwd_amd as sa

    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty((0,), dtype=torch.int32, device=DEV)
    logp, lse = sa.token_logps_fwd(x, ids)
    gx = sa.token_logps_bwd(x, ids, lse, torch.empty((0,), device=DEV))
    assert logp.shape == (0,) and gx.shape == (0, 64)


def test_full_vocabulary_sampled_rows():
    """8192 positions over a 201,088-entry vocabulary (the benchmarked size),
    checked against the oracle on sampled rows."""
    import attention_sink_fwd_amd as sa

    rows, vocab = 8192, 201088
    say(f"logps full size rows={rows} V={vocab}")
    d = make_logits_device(rows, vocab, "bf16", seed=15, device=DEV)
    logp, lse = sa.token_logps_fwd(d["logits"], d["ids"])
    gx = sa.token_logps_bwd(d["logits"], d["ids"], lse, d["grad"])
    torch.cuda.synchronize()
    pick = torch.tensor([0, 1, 777, 4095, 4096, 6000, 8190, 8191])
    x_cpu = d["logits"][pick.to(DEV)].cpu()
    ids_cpu = d["ids"][pick.to(DEV)].cpu()
    g_cpu = d["grad"][pick.to(DEV)].cpu()
    _check_fwd(logp[pick.to(DEV)], lse[pick.to(DEV)], x_cpu, ids_cpu, "full size")
    _check_grad(gx[pick.to(DEV)], x_cpu, ids_cpu, g_cpu, "bf16", "full size")
    # every row: log-probabilities are <= 0, and since softmax sums to one
    # each gradient row sums to ~0 (bf16 rounding of each entry aside)
    assert torch.isfinite(logp).all() and (logp <= 0).all()
    rowsum = gx.float().sum(dim=1).abs()
    assert (rowsum <= 2.0 ** -7 * d["grad"].abs() + 1e-6).all()
