"""SINK_ATTN_VALIDATE=1: the host copies the device-side index arrays and
rejects inconsistent ones with a status before anything is launched."""
import pytest
import torch

from synthetic.workloads import custom_workload, make_inputs, make_paged
from tests.parity_util import say

pytestmark = pytest.mark.gpu


def _status(fn):
    import attention_sink_fwd_amd as sa

    try:
        fn()
    except sa.SinkAttnError as e:
        return e.status
    return 0


@pytest.mark.parametrize("bad", ["first_not_zero", "decreasing", "over_max", "last_not_total"])
def test_validate_rejects_bad_cu_seqlens(monkeypatch, bad):
    import attention_sink_fwd_amd as sa
    from attention_sink_fwd_amd import _lib

    monkeypatch.setenv("SINK_ATTN_VALIDATE", "1")
    w = custom_workload((40, 30), 4, 2, 64, 0, "bf16")
    d = {k: v.to("cuda:0") for k, v in make_inputs(w, seed=3).items()}
    cu = {"first_not_zero": [1, 40, 70], "decreasing": [0, 50, 40], "over_max": [0, 10, 70],
          "last_not_total": [0, 40, 69]}[bad]
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
    say("case validate cu_seqlens", bad, cu)
    st = _status(lambda: sa.sink_attn_fwd(d["q"], d["k"], d["v"], d["sinks"], cu_t, 40))
    assert st == _lib.SINK_ATTN_ERR_INVALID_ARG
    # the same arrays are fine without the host check's complaint once corrected
    assert _status(lambda: sa.sink_attn_fwd(d["q"], d["k"], d["v"], d["sinks"], d["cu_seqlens"],
                                            40)) == 0


@pytest.mark.parametrize("bad", ["kv_len_below_q_len", "kv_len_past_table", "page_id_negative",
                                 "page_id_too_large"])
def test_validate_rejects_bad_paged_arrays(monkeypatch, bad):
    import attention_sink_fwd_amd as sa
    from attention_sink_fwd_amd import _lib

    monkeypatch.setenv("SINK_ATTN_VALIDATE", "1")
    w = custom_workload((130, 70), 4, 2, 64, 0, "bf16")
    pg = make_paged(make_inputs(w, seed=4), (3, 70), 64, seed=2)
    lens, bt = pg["kv_lens"].clone(), pg["block_table"].clone()
    if bad == "kv_len_below_q_len":
        lens[1] = 60
    elif bad == "kv_len_past_table":
        lens[0] = 64 * bt.shape[1] + 1
    elif bad == "page_id_negative":
        bt[0, 1] = -1
    else:
        bt[1, 0] = pg["k_cache"].shape[0]
    say("case validate paged", bad)
    dev = {k: v.to("cuda:0") for k, v in pg.items() if k != "rows"}

    def call(lens_t, bt_t):
        return lambda: sa.sink_attn_fwd_paged(dev["q"], dev["k_cache"], dev["v_cache"], bt_t, lens_t,
                                              dev["sinks"], dev["cu_seqlens"], 70)

    assert _status(call(lens.to("cuda:0"), bt.to("cuda:0"))) == _lib.SINK_ATTN_ERR_INVALID_ARG
    assert _status(call(dev["kv_lens"], dev["block_table"])) == 0
