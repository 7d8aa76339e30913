"""Pins of the float64 oracle against things other than itself (CPU only).

The oracle (oracle/sink_attention.py) writes sink attention out from its
definition.  Here it is pinned to:

* torch's scaled_dot_product_attention on the CPU in float64 -- a library
  softmax-attention routine -- with the sink emulated as one extra key
  column: a zero key, the additive mask entry S_h in that column, and a
  value vector that is zero except for one extra coordinate, which then
  carries p_sink.  GQA comes from the routine's own ``enable_gqa`` and the
  window from a band mask built here; its autograd gives dQ, dK, dV and,
  through the mask column, dS_h;
* central finite differences of L = sum(O * dO);
* closed forms: S_h = -inf (plain causal attention, the routine's own
  ``is_causal``), S_h large, q = 0, a length-1 sequence, window 1, and a
  small example whose exact values are rationals;
* invariants: packing sequences, GQA vs. repeated MHA, window >= L.

A planted mistake in the oracle (dropped sink, sign flip, wrong head map,
window off by one) makes at least one of these fail; see the mutation tests
at the end.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import sink_attention as osa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inputs(lengths, hq, hkv, d, seed, sink_value=None):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    q = rng.standard_normal((T, hq, d))
    k = rng.standard_normal((T, hkv, d))
    v = rng.standard_normal((T, hkv, d))
    do = rng.standard_normal((T, hq, d))
    s = rng.standard_normal(hq) if sink_value is None else np.full(hq, float(sink_value))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return q, k, v, do, s, cu


def _band_mask(L, window):
    """Visible[i, j] for local positions, built with torch.tril only."""
    ones = torch.ones(L, L, dtype=torch.bool)
    vis = torch.tril(ones)
    if window > 0:
        vis &= ~torch.tril(ones, diagonal=-window)
    return vis


def sdpa_with_sink_column(q, k, v, do, s, cu, scale, window):
    """Library reference: O, LSE, dQ, dK, dV, dS via torch SDPA + autograd."""
    T, hq, d = q.shape
    hkv = k.shape[1]
    O = np.zeros((T, hq, d))
    LSE = np.zeros((hq, T))
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    dS = np.zeros(hq)
    for b, e in zip(cu[:-1], cu[1:]):
        L = int(e - b)
        if L == 0:
            continue
        tq = torch.tensor(q[b:e]).permute(1, 0, 2)[None].clone().requires_grad_(True)
        tk = torch.tensor(k[b:e]).permute(1, 0, 2)[None].clone().requires_grad_(True)
        tv = torch.tensor(v[b:e]).permute(1, 0, 2)[None].clone().requires_grad_(True)
        k_ext = torch.cat([tk, torch.zeros(1, hkv, 1, d, dtype=torch.float64)], dim=2)
        v_ext = torch.cat([
            torch.cat([tv, torch.zeros(1, hkv, L, 1, dtype=torch.float64)], dim=3),
            torch.cat([torch.zeros(1, hkv, 1, d, dtype=torch.float64),
                       torch.ones(1, hkv, 1, 1, dtype=torch.float64)], dim=3),
        ], dim=2)
        vis = _band_mask(L, window)
        base = torch.zeros(L, L, dtype=torch.float64).masked_fill(~vis, float("-inf"))
        sink_col = torch.tensor(s, dtype=torch.float64).view(1, hq, 1, 1).expand(1, hq, L, 1)
        sink_col = sink_col.clone().requires_grad_(True)
        mask = torch.cat([base.view(1, 1, L, L).expand(1, hq, L, L), sink_col], dim=3)
        out = F.scaled_dot_product_attention(tq, k_ext, v_ext, attn_mask=mask,
                                             scale=scale, enable_gqa=True)
        tdo = torch.tensor(do[b:e]).permute(1, 0, 2)[None]
        (out[..., :d] * tdo).sum().backward()
        O[b:e] = out[0, :, :, :d].permute(1, 0, 2).detach().numpy()
        p_sink = out[0, :, :, d].detach().numpy()  # [hq, L]
        with np.errstate(divide="ignore", invalid="ignore"):
            LSE[:, b:e] = s[:, None] - np.log(p_sink)
        dQ[b:e] = tq.grad[0].permute(1, 0, 2).numpy()
        dK[b:e] = tk.grad[0].permute(1, 0, 2).numpy()
        dV[b:e] = tv.grad[0].permute(1, 0, 2).numpy()
        dS += sink_col.grad[0, :, :, 0].sum(dim=1).numpy()
    return O, LSE, dQ, dK, dV, dS


CASES = [
    # lengths, hq, hkv, d, window
    ((7,), 1, 1, 4, 0),
    ((13,), 4, 2, 8, 0),
    ((9, 0, 1, 17), 8, 1, 5, 0),
    ((20,), 4, 4, 6, 3),
    ((11, 5), 6, 2, 4, 1),
    ((33,), 2, 1, 16, 40),
    ((40, 3), 8, 8, 3, 7),
]


def _rel(a, b):
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (den if den > 0 else 1.0)


@pytest.mark.parametrize("lengths,hq,hkv,d,window", CASES)
def test_forward_and_backward_match_sdpa_with_sink_column(lengths, hq, hkv, d, window):
    q, k, v, do, s, cu = _inputs(lengths, hq, hkv, d, seed=hash((lengths, hq, d)) % 1000)
    s = s * 2.0  # spread the sinks so some rows are sink-dominated
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.forward(q, k, v, s, cu, scale, window, row_block=5)
    dq, dk, dv, ds = oracle.backward(q, k, v, s, do, cu, scale, window, row_block=5)
    O, LSE, dQ, dK, dV, dS = sdpa_with_sink_column(q, k, v, do, s, cu, scale, window)
    assert np.max(np.abs(o - O)) < 1e-12
    assert np.max(np.abs(lse - LSE)) < 1e-10
    assert _rel(dq, dQ) < 1e-12 and _rel(dk, dK) < 1e-12 and _rel(dv, dV) < 1e-12
    assert np.max(np.abs(ds - dS)) < 1e-11 * max(1.0, np.max(np.abs(dS)))


def test_sink_minus_inf_is_standard_causal_attention():
    lengths, hq, hkv, d = (24,), 8, 2, 8
    q, k, v, do, s, cu = _inputs(lengths, hq, hkv, d, seed=3, sink_value=-np.inf)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.forward(q, k, v, s, cu, scale)
    dq, dk, dv, ds = oracle.backward(q, k, v, s, do, cu, scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.all(ds == 0.0)
    tq = torch.tensor(q).permute(1, 0, 2)[None].requires_grad_(True)
    tk = torch.tensor(k).permute(1, 0, 2)[None].requires_grad_(True)
    tv = torch.tensor(v).permute(1, 0, 2)[None].requires_grad_(True)
    out = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale, enable_gqa=True)
    (out * torch.tensor(do).permute(1, 0, 2)[None]).sum().backward()
    assert np.max(np.abs(o - out[0].permute(1, 0, 2).detach().numpy())) < 1e-12
    assert _rel(dq, tq.grad[0].permute(1, 0, 2).numpy()) < 1e-12
    assert _rel(dk, tk.grad[0].permute(1, 0, 2).numpy()) < 1e-12
    assert _rel(dv, tv.grad[0].permute(1, 0, 2).numpy()) < 1e-12


def test_finite_differences_all_parameters():
    """Central differences (h = 1e-6) of L = sum(O * dO) w.r.t. every input."""
    for window in (0, 2):
        lengths, hq, hkv, d = (4, 3), 2, 1, 3
        q, k, v, do, s, cu = _inputs(lengths, hq, hkv, d, seed=11 + window)
        scale = 0.7
        dq, dk, dv, ds = oracle.backward(q, k, v, s, do, cu, scale, window)

        def loss(q_, k_, v_, s_):
            o, _ = oracle.forward(q_, k_, v_, s_, cu, scale, window)
            return float(np.sum(o * do))

        h = 1e-6
        for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("s", s, ds)):
            fd = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                args = {"q": q, "k": k, "v": v, "s": s}
                plus = arr.copy(); plus[idx] += h
                minus = arr.copy(); minus[idx] -= h
                args[name] = plus
                lp = loss(args["q"], args["k"], args["v"], args["s"])
                args[name] = minus
                lm = loss(args["q"], args["k"], args["v"], args["s"])
                fd[idx] = (lp - lm) / (2 * h)
            err = np.max(np.abs(fd - grad)) / max(1e-3, np.max(np.abs(grad)))
            assert err < 1e-6, (name, window, err)


def test_sink_large_drives_output_to_zero():
    lengths, hq, hkv, d = (16,), 2, 1, 8
    q, k, v, do, s, cu = _inputs(lengths, hq, hkv, d, seed=5, sink_value=30.0)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.forward(q, k, v, s, cu, scale)
    dq, dk, dv, ds = oracle.backward(q, k, v, s, do, cu, scale)
    # every logit here is far below 30, so each P_ij <= exp(x_ij - 30)
    x_max = np.max(np.abs(scale * np.einsum("thd,tgd->th", q, k[:, [0, 0]]))) + 10
    bound = math.exp(x_max - 30.0) * 16
    assert np.max(np.abs(o)) < bound * np.max(np.abs(v))
    assert np.max(np.abs(lse - 30.0)) < bound
    for g in (dq, dk, dv, ds):
        assert np.max(np.abs(g)) < 1e-6


@pytest.mark.parametrize("window", [0, 3])
def test_zero_queries_closed_form(window):
    """q = 0: every visible logit is 0, so O_i = sum v_j / (n_i + e^S)."""
    lengths, hq, hkv, d = (9, 4), 2, 2, 5
    _, k, v, _, s, cu = _inputs(lengths, hq, hkv, d, seed=7)
    q = np.zeros((sum(lengths), hq, d))
    o, lse = oracle.forward(q, k, v, s, cu, 0.5, window)
    for b, e in zip(cu[:-1], cu[1:]):
        for i in range(e - b):
            lo = 0 if window == 0 else max(0, i - window + 1)
            n = i + 1 - lo
            for h in range(hq):
                den = n + math.exp(s[h])
                np.testing.assert_allclose(o[b + i, h], v[b + lo:b + i + 1, h].sum(0) / den, atol=1e-14)
                assert abs(lse[h, b + i] - math.log(den)) < 1e-14


def _sigmoid(z):
    return 1.0 / (1.0 + math.exp(-z))


def test_length_one_and_window_one_closed_form():
    """Each row sees only its own key: O = sigmoid(x - S) v, dS = -s(1-s) dO.v."""
    for lengths, window in (((1, 1, 1), 0), ((6,), 1)):
        hq, hkv, d = 2, 1, 4
        q, k, v, do, s, cu = _inputs(lengths, hq, hkv, d, seed=13)
        scale = 0.5
        o, lse = oracle.forward(q, k, v, s, cu, scale, window)
        _, _, dv, ds = oracle.backward(q, k, v, s, do, cu, scale, window)
        want_ds = np.zeros(hq)
        for t in range(sum(lengths)):
            for h in range(hq):
                x = scale * q[t, h] @ k[t, 0]
                sg = _sigmoid(x - s[h])
                np.testing.assert_allclose(o[t, h], sg * v[t, 0], atol=1e-14)
                assert abs(lse[h, t] - np.logaddexp(x, s[h])) < 1e-13
                want_ds[h] += -sg * (1 - sg) * (do[t, h] @ v[t, 0])
        np.testing.assert_allclose(ds, want_ds, rtol=1e-12, atol=1e-14)
        # dV_j = sum over the group's heads of sigmoid(x - S) dO
        want_dv = np.zeros_like(dv)
        for t in range(sum(lengths)):
            for h in range(hq):
                want_dv[t, 0] += _sigmoid(scale * q[t, h] @ k[t, 0] - s[h]) * do[t, h]
        np.testing.assert_allclose(dv, want_dv, atol=1e-13)


def test_hand_example_exact_rationals():
    """Fixture tests/golden/hand_example.json: exact values derived by hand."""
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float64).reshape(-1, 1, 1)
    k = np.log(np.array(g["exp_k"], dtype=np.float64)).reshape(-1, 1, 1)
    v = np.array(g["v"], dtype=np.float64).reshape(-1, 1, 1)
    do = np.array(g["dout"], dtype=np.float64).reshape(-1, 1, 1)
    s = np.log(np.array([g["exp_sink"]], dtype=np.float64))
    cu = np.array([0, len(g["v"])])
    o, lse = oracle.forward(q, k, v, s, cu, 1.0)
    dq, dk, dv, ds = oracle.backward(q, k, v, s, do, cu, 1.0)

    def frac(x):
        return float(x[0]) / float(x[1])

    np.testing.assert_allclose(o[:, 0, 0], [frac(x) for x in g["o"]], rtol=1e-14)
    np.testing.assert_allclose(np.exp(lse[0]), [frac(x) for x in g["exp_lse"]], rtol=1e-14)
    np.testing.assert_allclose(dv[:, 0, 0], [frac(x) for x in g["dv"]], rtol=1e-14)
    np.testing.assert_allclose(ds, [frac(g["dsink"])], rtol=1e-14)


def test_window_at_least_length_equals_plain_causal():
    lengths, hq, hkv, d = (10, 6), 4, 2, 4
    q, k, v, do, s, cu = _inputs(lengths, hq, hkv, d, seed=17)
    a = oracle.forward(q, k, v, s, cu, 0.4, 0)
    b = oracle.forward(q, k, v, s, cu, 0.4, 10)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    ga = oracle.backward(q, k, v, s, do, cu, 0.4, 0)
    gb = oracle.backward(q, k, v, s, do, cu, 0.4, 12)
    for x, y in zip(ga, gb):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-14)


def test_packing_equals_separate_runs():
    lengths, hq, hkv, d = (5, 0, 12, 1, 7), 4, 2, 6
    q, k, v, do, s, cu = _inputs(lengths, hq, hkv, d, seed=19)
    o, lse = oracle.forward(q, k, v, s, cu, 0.3, 4)
    g = oracle.backward(q, k, v, s, do, cu, 0.3, 4)
    for b, e in zip(cu[:-1], cu[1:]):
        sl = slice(b, e)
        c1 = np.array([0, e - b])
        o1, l1 = oracle.forward(q[sl], k[sl], v[sl], s, c1, 0.3, 4)
        np.testing.assert_allclose(o[sl], o1, atol=1e-15)
        np.testing.assert_allclose(lse[:, sl], l1, atol=1e-15)
        g1 = oracle.backward(q[sl], k[sl], v[sl], s, do[sl], c1, 0.3, 4)
        for x, y in zip(g[:3], g1[:3]):
            np.testing.assert_allclose(x[sl], y, atol=1e-14)
    # dS sums over sequences
    total = sum(oracle.backward(q[b:e], k[b:e], v[b:e], s, do[b:e], np.array([0, e - b]), 0.3, 4)[3]
                for b, e in zip(cu[:-1], cu[1:]))
    np.testing.assert_allclose(g[3], total, rtol=1e-13, atol=1e-15)


def test_gqa_equals_repeated_mha():
    lengths, hq, hkv, d = (14,), 6, 2, 5
    q, k, v, do, s, cu = _inputs(lengths, hq, hkv, d, seed=23)
    rep = hq // hkv
    k_rep = np.repeat(k, rep, axis=1)
    v_rep = np.repeat(v, rep, axis=1)
    o, lse = oracle.forward(q, k, v, s, cu, 0.45)
    o2, lse2 = oracle.forward(q, k_rep, v_rep, s, cu, 0.45)
    np.testing.assert_allclose(o, o2, atol=1e-15)
    np.testing.assert_allclose(lse, lse2, atol=1e-15)
    dq, dk, dv, ds = oracle.backward(q, k, v, s, do, cu, 0.45)
    dq2, dk2, dv2, ds2 = oracle.backward(q, k_rep, v_rep, s, do, cu, 0.45)
    np.testing.assert_allclose(dq, dq2, atol=1e-14)
    np.testing.assert_allclose(dk, dk2.reshape(-1, hkv, rep, d).sum(2), atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(-1, hkv, rep, d).sum(2), atol=1e-13)
    np.testing.assert_allclose(ds, ds2, atol=1e-14)


def test_row_and_key_helpers_match_full_computation():
    lengths, hq, hkv, d = (30, 17), 4, 2, 8
    for window in (0, 6):
        q, k, v, do, s, cu = _inputs(lengths, hq, hkv, d, seed=29 + window)
        o, lse = oracle.forward(q, k, v, s, cu, 0.35, window)
        dq, dk, dv, _ = oracle.backward(q, k, v, s, do, cu, 0.35, window)
        rows = np.array([0, 1, 5, 16])
        for seq in (0, 1):
            b = cu[seq]
            for h in (0, 3):
                o_r, l_r = oracle.forward_rows(q, k, v, s, cu, 0.35, window, seq, h, rows)
                np.testing.assert_allclose(o_r, o[b + rows, h], atol=1e-14)
                np.testing.assert_allclose(l_r, lse[h, b + rows], atol=1e-13)
                dq_r = oracle.backward_rows(q, k, v, s, do, cu, 0.35, window, seq, h, rows)
                np.testing.assert_allclose(dq_r, dq[b + rows, h], atol=1e-13)
            keys = np.array([0, 3, 12, 16])
            for g in range(hkv):
                dk_k, dv_k = oracle.backward_keys(q, k, v, s, do, cu, 0.35, window, seq, g, keys)
                np.testing.assert_allclose(dk_k, dk[b + keys, g], atol=1e-13)
                np.testing.assert_allclose(dv_k, dv[b + keys, g], atol=1e-13)


@pytest.mark.parametrize("window,sink_value", [(0, None), (6, None), (0, -math.inf), (3, 30.0)])
def test_blocked_key_helper_matches_backward_and_sdpa(window, sink_value):
    """backward_keys_blocked: dK, dV at a key set and the per-sequence sink
    gradients, against backward and directly against the SDPA reference."""
    lengths, hq, hkv, d = (45, 0, 70), 6, 2, 8
    q, k, v, do, s, cu = _inputs(lengths, hq, hkv, d, seed=37 + window, sink_value=sink_value)
    scale = 0.4
    dq, dk, dv, ds = oracle.backward(q, k, v, s, do, cu, scale, window)
    _, _, _, dK, dV, dS = sdpa_with_sink_column(q, k, v, do, s, cu, scale, window)
    ds_sum = np.zeros(hq)
    for seq in range(len(lengths)):
        b, L = int(cu[seq]), int(lengths[seq])
        keys = np.array([j for j in (0, 1, 7, 31, 44, 69) if j < L], dtype=np.int64)
        for g in range(hkv):
            dk_k, dv_k, ds_g = oracle.backward_keys_blocked(q, k, v, s, do, cu, scale, window, seq, g,
                                                             keys, row_block=16)
            np.testing.assert_allclose(dk_k, dk[b + keys, g], atol=1e-13)
            np.testing.assert_allclose(dv_k, dv[b + keys, g], atol=1e-13)
            np.testing.assert_allclose(dk_k, dK[b + keys, g], atol=1e-11)
            np.testing.assert_allclose(dv_k, dV[b + keys, g], atol=1e-11)
            for h, val in ds_g.items():
                ds_sum[h] += val
    np.testing.assert_allclose(ds_sum, ds, atol=1e-13)
    np.testing.assert_allclose(ds_sum, dS, atol=1e-11)
    # a head subset and an empty key set give the same sink gradients
    _, _, ds_one = oracle.backward_keys_blocked(q, k, v, s, do, cu, scale, window, 2, 1, [], heads=[4])
    _, _, ds_all = oracle.backward_keys_blocked(q, k, v, s, do, cu, scale, window, 2, 1, [0, 5])
    assert ds_one[4] == pytest.approx(ds_all[4], abs=1e-14)


# ---------------------------------------------------------------------------
# Planted mistakes: each mutated oracle must fail at least one pin above.


def _pin_sdpa_fails():
    lengths, hq, hkv, d, window = (12, 5), 4, 2, 4, 3
    q, k, v, do, s, cu = _inputs(lengths, hq, hkv, d, seed=31)
    scale = 0.5
    o, lse = oracle.forward(q, k, v, s, cu, scale, window)
    dq, dk, dv, ds = oracle.backward(q, k, v, s, do, cu, scale, window)
    O, LSE, dQ, dK, dV, dS = sdpa_with_sink_column(q, k, v, do, s, cu, scale, window)
    ok = (np.max(np.abs(o - O)) < 1e-12 and np.max(np.abs(lse - LSE)) < 1e-10
          and _rel(dq, dQ) < 1e-12 and _rel(dk, dK) < 1e-12 and _rel(dv, dV) < 1e-12
          and np.max(np.abs(ds - dS)) < 1e-11)
    return not ok


def test_planted_mistakes_are_caught(monkeypatch):
    orig_probs = osa._row_probabilities
    orig_vis = osa._visibility
    orig_range = osa.visible_key_range

    def no_sink(qh, kg, sink, rows, scale, window):
        return orig_probs(qh, kg, -np.inf, rows, scale, window)

    def sink_scaled(qh, kg, sink, rows, scale, window):
        return orig_probs(qh, kg, sink * scale, rows, scale, window)

    def window_off_by_one(rows, keys, window):
        return orig_vis(rows, keys, window + 1 if window else 0)

    def range_off_by_one(i, window):
        lo, hi = orig_range(i, window + 1 if window else 0)
        return lo, hi

    mutations = [
        ("_row_probabilities", no_sink),
        ("_row_probabilities", sink_scaled),
        ("_visibility", window_off_by_one),
        ("kv_head_of", lambda h, a, b: h % b),
    ]
    assert not _pin_sdpa_fails()
    for attr, fn in mutations:
        monkeypatch.setattr(osa, attr, fn)
        if attr == "_visibility":
            monkeypatch.setattr(osa, "visible_key_range", range_off_by_one)
        assert _pin_sdpa_fails(), attr
        monkeypatch.undo()
    assert not _pin_sdpa_fails()


def test_planted_sign_flip_in_sink_gradient_is_caught(monkeypatch):
    """A flipped dS_h sign passes the forward pins but not finite differences."""
    lengths, hq, hkv, d = (5,), 2, 1, 3
    q, k, v, do, s, cu = _inputs(lengths, hq, hkv, d, seed=37)
    orig_backward = oracle.backward

    def flipped(*a, **kw):
        dq, dk, dv, ds = orig_backward(*a, **kw)
        return dq, dk, dv, -ds

    ds = flipped(q, k, v, s, do, cu, 0.6)[3]
    h = 1e-6
    fd = np.zeros(hq)
    for i in range(hq):
        sp, sm = s.copy(), s.copy()
        sp[i] += h
        sm[i] -= h
        fd[i] = (np.sum(oracle.forward(q, k, v, sp, cu, 0.6)[0] * do)
                 - np.sum(oracle.forward(q, k, v, sm, cu, 0.6)[0] * do)) / (2 * h)
    assert np.max(np.abs(fd - ds)) > 1e-3
    assert np.max(np.abs(fd - orig_backward(q, k, v, s, do, cu, 0.6)[3])) < 1e-8


# ---- paged-cache forward (new tokens at the end of a cached context) ----

from synthetic.workloads import custom_workload, make_inputs, make_paged  # noqa: E402


@pytest.mark.parametrize("lengths,q_lens,page_size,window", [
    ((70, 5, 129), (70, 5, 129), 64, 0),     # whole sequences: the plain forward
    ((70, 5, 129), (1, 5, 40), 64, 0),       # decode, whole, prefill of 40
    ((200, 90), (17, 1), 128, 33),           # window, other page size
])
def test_paged_forward_equals_forward_rows(lengths, q_lens, page_size, window):
    w = custom_workload(lengths, 4, 2, 16, window, "f32")
    inp = make_inputs(w, seed=11)
    pg = make_paged(inp, q_lens, page_size, seed=3)
    o_ref, lse_ref = osa.forward(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["cu_seqlens"],
                                 w.softmax_scale, window)
    o, lse = osa.forward_paged(pg["q"], pg["k_cache"], pg["v_cache"], pg["block_table"],
                               pg["kv_lens"], pg["sinks"], pg["cu_seqlens"], w.softmax_scale, window)
    rows = pg["rows"].numpy()
    assert np.abs(o - o_ref[rows]).max() < 1e-12
    assert np.abs(lse - lse_ref[:, rows]).max() < 1e-12


def test_paged_gather_follows_the_block_table():
    w = custom_workload((130, 64), 2, 1, 8, 0, "f32")
    inp = make_inputs(w, seed=2)
    a = make_paged(inp, (130, 64), 64, seed=1)
    b = make_paged(inp, (130, 64), 64, seed=9)  # other page order, same sequences
    assert not torch.equal(a["block_table"], b["block_table"])
    for s, (b0, L) in enumerate(((0, 130), (130, 64))):
        ga = osa.gather_paged(a["k_cache"], a["block_table"], L, s)
        gb = osa.gather_paged(b["v_cache"], b["block_table"], L, s)
        assert np.array_equal(ga, inp["k"][b0:b0 + L].double().numpy())
        assert np.array_equal(gb, inp["v"][b0:b0 + L].double().numpy())


def test_paged_single_key_closed_form():
    # kv_len = q_len = 1: O = sigmoid(x - S) v0, LSE = logaddexp(S, x), x = tau q.k
    q = torch.tensor([[[0.5, -1.0, 2.0, 0.25]]])
    k_cache = torch.full((2, 64, 1, 4), float("nan"))
    v_cache = torch.full((2, 64, 1, 4), float("nan"))
    k_cache[1, 0, 0] = torch.tensor([1.0, 0.5, -0.5, 2.0])
    v_cache[1, 0, 0] = torch.tensor([3.0, -2.0, 1.0, 0.5])
    bt = torch.tensor([[1, -1]], dtype=torch.int32)
    sinks = torch.tensor([0.3])
    tau = 0.5
    o, lse = osa.forward_paged(q, k_cache, v_cache, bt, torch.tensor([1], dtype=torch.int32), sinks,
                               torch.tensor([0, 1], dtype=torch.int32), tau, 0)
    x = tau * float(q[0, 0].double() @ k_cache[1, 0, 0].double())
    sv = float(sinks[0])  # the float32 value the oracle receives
    p = 1.0 / (1.0 + math.exp(sv - x))
    assert np.allclose(o[0, 0], p * v_cache[1, 0, 0].double().numpy(), atol=1e-15)
    assert abs(lse[0, 0] - np.logaddexp(sv, x)) < 1e-15
