"""Seeded random shapes, bf16 and head_dim 64 (the matrix-core path), forward
and backward against the float64 oracle on every element.

Each case draws from its own seed: one to five sequences of 0..2099 tokens
(one of them sometimes set to a tile-boundary length such as 1, 63, 65,
127, 129 or 257; at most two sequences when a KV head has 32 or 64 query
heads), 1, 2 or 4 KV heads with 1..64 query heads each, no window, a window
of 1..139 keys (the fused short-window backward takes up to 128) or of
140..899 keys, and sinks drawn normally, mixed with -inf and +30, all -inf
or all +30.  The shapes combine what the fixed cases cover one at a time:
ragged tails in several sequences at once, one-token sequences between long
ones, every head-packing factor, and windows on both sides of the fused
kernel's limit.
"""
import math

import numpy as np
import pytest

from synthetic.workloads import custom_workload, make_inputs
from tests.parity_util import check_full, run_gpu, say
from tests.test_gpu_parity import _oracle_full, _set_sinks

pytestmark = pytest.mark.gpu

SEEDS = range(5000, 5048)


def draw_shape(seed):
    rng = np.random.default_rng(seed)
    nseq = int(rng.integers(1, 6))
    lens = [int(x) for x in rng.integers(0, 2100, size=nseq)]
    if rng.random() < 0.2:
        lens[int(rng.integers(0, nseq))] = int(rng.choice([1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257]))
    if sum(lens) == 0:
        lens[0] = 1
    hkv = int(rng.choice([1, 2, 4]))
    grp = int(rng.choice([1, 2, 3, 4, 6, 8, 16, 32, 64]))
    if grp >= 32:
        hkv = 1
        nseq = min(nseq, 2)
        lens = lens[:nseq]
        if sum(lens) == 0:
            lens[0] = 1
    r = rng.random()
    window = 0 if r < 0.3 else int(rng.integers(1, 140)) if r < 0.85 else int(rng.integers(140, 900))
    sinks = str(rng.choice(["normal", "normal", "mixed", "minus_inf", "plus30"]))
    return lens, hkv * grp, hkv, window, sinks


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape_matches_oracle(seed):
    lens, hq, hkv, window, sinks = draw_shape(seed)
    label = f"seed {seed} L={lens} hq={hq} hkv={hkv} W={window} sinks={sinks}"
    say("case", label)
    w = custom_workload(lens, hq, hkv, 64, window, "bf16")
    inp = _set_sinks(make_inputs(w, seed=seed), sinks, hq)
    scale = 1.0 / math.sqrt(64)
    gpu = run_gpu(inp, w.max_seqlen, scale, window)
    check_full(gpu, _oracle_full(inp, scale, window), label)
    if sinks == "minus_inf":
        assert np.all(gpu["ds"] == 0.0)
