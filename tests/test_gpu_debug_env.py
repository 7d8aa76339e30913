"""The launch debugging switches of the library (SINK_ATTN_TRACE,
SINK_ATTN_SYNC_DEBUG): every kernel launch of a forward + backward prints
its line, and with a synchronisation after every launch the results are
those of the oracle, as without."""
import math

import pytest

from synthetic.workloads import custom_workload, make_inputs
from tests.parity_util import check_full, run_gpu, say
from tests.test_gpu_parity import _oracle_full

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("window,expect", [
    (0, ("fwd_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel", "bwd_post_kernel")),
    (64, ("fwd_kernel", "bwd_window_kernel", "bwd_window_post_kernel")),
])
def test_trace_and_sync_debug(monkeypatch, capfd, window, expect):
    monkeypatch.setenv("SINK_ATTN_TRACE", "1")
    monkeypatch.setenv("SINK_ATTN_SYNC_DEBUG", "1")
    w = custom_workload((300, 70), 8, 2, 64, window, "bf16")
    inp = make_inputs(w, seed=31 + window)
    say("case trace + sync debug, window", window)
    gpu = run_gpu(inp, w.max_seqlen, 1.0 / math.sqrt(64), window)
    err = capfd.readouterr().err
    lines = [l for l in err.splitlines() if l.startswith("[sink_attn] launch ")]
    for name in expect:
        assert any(f" {name}" in l for l in lines), (name, lines)
    assert all("(launch failed)" not in l for l in lines)
    check_full(gpu, _oracle_full(inp, 1.0 / math.sqrt(64), window), f"debug env W={window}")
