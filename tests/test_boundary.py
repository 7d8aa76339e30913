"""The C ABI without a GPU: the library loads, exports what the header
declares, and rejects every bad argument before anything is enqueued."""
import ctypes
import os
import re

import pytest

from attention_sink_fwd_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def _declared_functions():
    names = set()
    for header in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
        # function declarations: a return type, then name( ... );
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = _lib.load()
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name
    # the symbols are plain C names (no C++ mangling)
    out = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    for name in declared:
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_status_strings():
    lib = _lib.load()
    seen = set()
    for st in range(5):
        s = lib.sink_attn_status_string(st).decode()
        assert s and s not in seen
        seen.add(s)
    assert lib.sink_attn_status_string(99).decode() == "unknown status"


def _good_params(T=128, hq=8, hkv=2, d=64, window=0, dtype=0):
    p = _lib.SinkAttnParams()
    p.cu_seqlens = 256  # never read by the host unless SINK_ATTN_VALIDATE=1
    p.num_seqs = 1
    p.max_seqlen = T
    p.total_tokens = T
    p.num_q_heads = hq
    p.num_kv_heads = hkv
    p.head_dim = d
    p.softmax_scale = 0.125
    p.causal = 1
    p.window = window
    p.dtype = dtype
    return p


FAKE = 1 << 20  # aligned, non-null, never dereferenced by the host


def _fwd(p, **override):
    lib = _lib.load()
    args = dict(q=FAKE, k=FAKE, v=FAKE, sinks=FAKE, o=FAKE, lse=FAKE)
    args.update(override)
    ptr = ctypes.byref(p) if p is not None else None
    return lib.sink_attn_fwd(ptr, args["q"], args["k"], args["v"], args["sinks"], args["o"],
                             args["lse"], None)


def _bwd(p, ws_bytes=None, **override):
    lib = _lib.load()
    args = dict(q=FAKE, k=FAKE, v=FAKE, sinks=FAKE, o=FAKE, lse=FAKE, dout=FAKE, dq=FAKE,
                dk=FAKE, dv=FAKE, dsinks=FAKE, ws=FAKE)
    args.update(override)
    if ws_bytes is None:
        ws_bytes = 1 << 40
    return lib.sink_attn_bwd(ctypes.byref(p), args["q"], args["k"], args["v"], args["sinks"],
                             args["o"], args["lse"], args["dout"], args["dq"], args["dk"],
                             args["dv"], args["dsinks"], args["ws"], ws_bytes, None)


@pytest.mark.parametrize("field,value,status", [
    ("num_seqs", 0, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("num_seqs", 70000, _lib.SINK_ATTN_ERR_UNSUPPORTED),
    ("total_tokens", -1, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("max_seqlen", 0, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("num_q_heads", 0, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("num_q_heads", 16384, _lib.SINK_ATTN_ERR_UNSUPPORTED),
    ("total_tokens", 1 << 26, _lib.SINK_ATTN_ERR_UNSUPPORTED),
    ("max_seqlen", 1 << 30, _lib.SINK_ATTN_ERR_UNSUPPORTED),
    ("num_kv_heads", 3, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("head_dim", 12, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("head_dim", 0, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("head_dim", 128, _lib.SINK_ATTN_ERR_UNSUPPORTED),
    ("softmax_scale", 0.0, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("softmax_scale", float("nan"), _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("softmax_scale", float("inf"), _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("causal", 0, _lib.SINK_ATTN_ERR_UNSUPPORTED),
    ("window", -1, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("dtype", 7, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("cu_seqlens", None, _lib.SINK_ATTN_ERR_INVALID_ARG),
])
def test_bad_params_are_rejected_without_launch(field, value, status):
    lib = _lib.load()
    p = _good_params()
    setattr(p, field, value)
    assert _fwd(p) == status
    assert lib.sink_attn_last_error().decode() != ""
    assert _bwd(p) == status
    assert lib.sink_attn_bwd_workspace_size(ctypes.byref(p)) == 0


@pytest.mark.parametrize("value", ["0", "3", "-2", "abc"])
def test_bad_dkdv_heads_override_is_rejected(monkeypatch, value):
    monkeypatch.setenv("SINK_ATTN_DKDV_HEADS", value)
    p = _good_params()
    assert _bwd(p) == _lib.SINK_ATTN_ERR_INVALID_ARG
    assert "SINK_ATTN_DKDV_HEADS" in _lib.load().sink_attn_last_error().decode()


@pytest.mark.parametrize("value", ["0", "5", "-1", "abc"])
def test_bad_fused_tiles_override_is_rejected(monkeypatch, value):
    monkeypatch.setenv("SINK_ATTN_FUSED_TILES", value)
    lib = _lib.load()
    p = _good_params(window=64)  # bf16, d 64, a window shorter than the sequence: the fused backward
    assert _bwd(p) == _lib.SINK_ATTN_ERR_INVALID_ARG
    assert "SINK_ATTN_FUSED_TILES" in lib.sink_attn_last_error().decode()
    assert lib.sink_attn_bwd_workspace_size(ctypes.byref(p)) == 0
    # without a window cut the fused kernel is not used and the variable is not read
    assert lib.sink_attn_bwd_workspace_size(ctypes.byref(_good_params())) > 0


def test_null_params():
    lib = _lib.load()
    assert _fwd(None) == _lib.SINK_ATTN_ERR_INVALID_ARG
    assert lib.sink_attn_bwd_workspace_size(None) == 0


@pytest.mark.parametrize("name", ["q", "k", "v", "sinks", "o", "lse"])
def test_fwd_null_tensor(name):
    assert _fwd(_good_params(), **{name: None}) == _lib.SINK_ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["q", "k", "v", "sinks", "o", "lse", "dout", "dq", "dk", "dv",
                                  "dsinks", "ws"])
def test_bwd_null_tensor(name):
    assert _bwd(_good_params(), **{name: None}) == _lib.SINK_ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["q", "k", "v", "o"])
def test_misaligned_tensor(name):
    assert _fwd(_good_params(), **{name: FAKE + 2}) == _lib.SINK_ATTN_ERR_INVALID_ARG


def test_workspace_size_and_too_small():
    lib = _lib.load()
    T, hq, hkv, d = 1000, 8, 2, 64
    p = _good_params(T, hq, hkv, d)
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # one dS partial per dQ tile and head; the dQ kernel packs the 4 heads of
    # a KV group, so a tile holds 128 / 4 rows
    parts = (T + 31) // 32
    # dK/dV partial sums: one plane per head group; this small shape takes one
    # head per group (P = hq / hkv planes); the scaled queries are bf16 [T, Hq, d]
    want = (2 * up(4 * hq * T) + up(2 * T * hq * d) + 2 * up(4 * (hq // hkv) * T * hkv * d)
            + up(4 * parts * hq))
    assert lib.sink_attn_bwd_workspace_size(ctypes.byref(p)) == want
    assert _bwd(p, ws_bytes=want - 1) == _lib.SINK_ATTN_ERR_WORKSPACE_TOO_SMALL
    assert "workspace" in lib.sink_attn_last_error().decode()
    assert _bwd(p, ws_bytes=want, ws=FAKE + 16) == _lib.SINK_ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("heads,planes", [(4, 0), (2, 2), (1, 4)])
def test_workspace_follows_dkdv_heads(monkeypatch, heads, planes):
    monkeypatch.setenv("SINK_ATTN_DKDV_HEADS", str(heads))
    lib = _lib.load()
    T, hq, hkv, d = 1000, 8, 2, 64
    p = _good_params(T, hq, hkv, d)
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    want = (2 * up(4 * hq * T) + up(2 * T * hq * d) + 2 * up(4 * planes * T * hkv * d)
            + up(4 * ((T + 31) // 32) * hq))
    assert lib.sink_attn_bwd_workspace_size(ctypes.byref(p)) == want


@pytest.mark.parametrize("window,dtype,fused_env,fused", [
    (128, 0, None, True), (1, 0, None, True), (129, 0, None, False), (128, 1, None, False),
    (128, 0, "0", False), (0, 0, None, False)])
def test_workspace_of_the_fused_short_window_path(monkeypatch, window, dtype, fused_env, fused):
    """bf16, head_dim 64 and a window of 1..128 keys take the fused kernel:
    two float dK/dV planes and one dS partial per (query head, 128-row tile);
    otherwise (or with SINK_ATTN_BWD_FUSED=0) the dQ and dK/dV kernels'
    workspace."""
    monkeypatch.delenv("SINK_ATTN_DKDV_HEADS", raising=False)
    monkeypatch.delenv("SINK_ATTN_PACK_HEADS", raising=False)
    if fused_env is None:
        monkeypatch.delenv("SINK_ATTN_BWD_FUSED", raising=False)
    else:
        monkeypatch.setenv("SINK_ATTN_BWD_FUSED", fused_env)
    lib = _lib.load()
    T, hq, hkv, d = 1000, 8, 2, 64
    p = _good_params(T, hq, hkv, d, window=window, dtype=dtype)
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    got = lib.sink_attn_bwd_workspace_size(ctypes.byref(p))
    fused_size = 2 * up(4 * 2 * T * hkv * d) + up(4 * ((T + 127) // 128) * hq)
    assert (got == fused_size) == fused, (got, fused_size)
    if not fused:
        assert got >= 2 * up(4 * hq * T) + up(2 * T * hq * d)


def test_fused_path_needs_at_most_64_heads_per_kv_head(monkeypatch):
    monkeypatch.delenv("SINK_ATTN_BWD_FUSED", raising=False)
    lib = _lib.load()
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    T, d = 300, 64
    for hq, fused in ((64, True), (128, False)):
        p = _good_params(T, hq, 1, d, window=100)
        got = lib.sink_attn_bwd_workspace_size(ctypes.byref(p))
        assert (got == 2 * up(4 * 2 * T * d) + up(4 * ((T + 127) // 128) * hq)) == fused


@pytest.mark.parametrize("pack,rows", [(1, 128), (2, 64), (4, 32)])
def test_workspace_follows_pack_heads(monkeypatch, pack, rows):
    monkeypatch.setenv("SINK_ATTN_PACK_HEADS", str(pack))
    monkeypatch.setenv("SINK_ATTN_DKDV_HEADS", "4")
    lib = _lib.load()
    T, hq, hkv, d = 1000, 8, 2, 64
    p = _good_params(T, hq, hkv, d)
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    want = 2 * up(4 * hq * T) + up(2 * T * hq * d) + up(4 * ((T + rows - 1) // rows) * hq)
    assert lib.sink_attn_bwd_workspace_size(ctypes.byref(p)) == want


def test_forward_with_no_tokens_is_a_no_op():
    p = _good_params(T=0)
    p.max_seqlen = 0
    assert _fwd(p, q=None, k=None, v=None, o=None, lse=None, sinks=None) == _lib.SINK_ATTN_OK


def test_package_raises_when_library_is_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load()


def test_set_bwd_events_accepts_partial_and_null():
    lib = _lib.load()
    try:
        arr = (ctypes.c_void_p * 4)(FAKE, FAKE, None, FAKE)  # NULL entries skip that point
        assert lib.sink_attn_set_bwd_events(arr) == _lib.SINK_ATTN_OK
        assert lib.sink_attn_set_bwd_events((ctypes.c_void_p * 4)()) == _lib.SINK_ATTN_OK
    finally:
        assert lib.sink_attn_set_bwd_events(None) == _lib.SINK_ATTN_OK


def _paged_kv(**override):
    kv = _lib.SinkAttnPagedKV()
    vals = dict(k_cache=FAKE, v_cache=FAKE, block_table=FAKE, kv_lens=FAKE, num_pages=4,
                page_size=64, max_blocks_per_seq=2)
    vals.update(override)
    for name, val in vals.items():
        setattr(kv, name, val)
    return kv


def _fwd_paged(p, kv, **override):
    lib = _lib.load()
    args = dict(q=FAKE, sinks=FAKE, o=FAKE, lse=FAKE)
    args.update(override)
    kvp = ctypes.byref(kv) if kv is not None else None
    return lib.sink_attn_fwd_paged(ctypes.byref(p), kvp, args["q"], args["sinks"], args["o"],
                                   args["lse"], None)


@pytest.mark.parametrize("field,value", [
    ("page_size", 0), ("page_size", 32), ("page_size", 96), ("num_pages", 0),
    ("max_blocks_per_seq", 0), ("k_cache", None), ("v_cache", None), ("block_table", None),
    ("kv_lens", None), ("k_cache", FAKE + 4),
])
def test_paged_forward_rejects_bad_cache_description(field, value):
    p = _good_params()
    assert _fwd_paged(p, _paged_kv(**{field: value})) == _lib.SINK_ATTN_ERR_INVALID_ARG
    assert _lib.load().sink_attn_last_error().decode() != ""


def test_paged_forward_rejects_null_kv_and_tensors():
    p = _good_params()
    assert _fwd_paged(p, None) == _lib.SINK_ATTN_ERR_INVALID_ARG
    for name in ("q", "sinks", "o", "lse"):
        assert _fwd_paged(p, _paged_kv(), **{name: None}) == _lib.SINK_ATTN_ERR_INVALID_ARG


def test_paged_forward_rejects_oversized_block_table_span():
    p = _good_params()
    kv = _paged_kv(page_size=1 << 20, max_blocks_per_seq=1 << 12)
    assert _fwd_paged(p, kv) == _lib.SINK_ATTN_ERR_UNSUPPORTED


def test_paged_forward_with_no_new_tokens_is_a_no_op():
    p = _good_params(T=0)
    p.max_seqlen = 0
    assert _fwd_paged(p, _paged_kv(k_cache=None, v_cache=None), q=None, o=None, lse=None,
                      sinks=None) == _lib.SINK_ATTN_OK


@pytest.mark.parametrize("value", ["0", "3", "64", "x"])
def test_bad_fwd_heads_override_is_rejected(monkeypatch, value):
    monkeypatch.setenv("SINK_ATTN_PACK_HEADS", value)
    p = _good_params()  # Hq/Hkv = 4
    assert _fwd(p) == _lib.SINK_ATTN_ERR_INVALID_ARG
    assert "SINK_ATTN_PACK_HEADS" in _lib.load().sink_attn_last_error().decode()
    assert _fwd_paged(p, _paged_kv()) == _lib.SINK_ATTN_ERR_INVALID_ARG



# ---- per-token log-probabilities ----

def _logps_fwd(**override):
    lib = _lib.load()
    a = dict(logits=FAKE, dtype=0, batch=2, seq=2, vocab=100, bstride=208, stride=104, ids=FAKE, logps=FAKE,
             lse=None)
    a.update(override)
    return lib.token_logps_fwd(a["logits"], a["dtype"], a["batch"], a["seq"], a["vocab"], a["bstride"],
                               a["stride"], a["ids"], a["logps"], a["lse"], None)


def _logps_bwd(**override):
    lib = _lib.load()
    a = dict(logits=FAKE, dtype=0, batch=2, seq=2, vocab=100, bstride=208, stride=104, ids=FAKE, lse=FAKE,
             g=FAKE, gx=FAKE, gbstride=208, gstride=104)
    a.update(override)
    return lib.token_logps_bwd(a["logits"], a["dtype"], a["batch"], a["seq"], a["vocab"], a["bstride"],
                               a["stride"], a["ids"], a["lse"], a["g"], a["gx"], a["gbstride"], a["gstride"],
                               None)


@pytest.mark.parametrize("field,value,status", [
    ("dtype", 3, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("batch", -1, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("seq", -1, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("seq", 1 << 23, _lib.SINK_ATTN_ERR_UNSUPPORTED),   # 2 x 2^23 rows
    ("vocab", 0, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("stride", 96, _lib.SINK_ATTN_ERR_INVALID_ARG),     # below vocab
    ("stride", 108, _lib.SINK_ATTN_ERR_INVALID_ARG),    # not a multiple of 8
    ("bstride", 212, _lib.SINK_ATTN_ERR_INVALID_ARG),   # not a multiple of 8
    ("bstride", -208, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("logits", None, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("logits", FAKE + 8, _lib.SINK_ATTN_ERR_INVALID_ARG),
    ("ids", None, _lib.SINK_ATTN_ERR_INVALID_ARG),
])
def test_logps_rejects_bad_arguments(field, value, status):
    assert _logps_fwd(**{field: value}) == status
    assert _lib.load().sink_attn_last_error().decode() != ""
    assert _logps_bwd(**{field: value}) == status


def test_logps_output_pointers_are_checked():
    assert _logps_fwd(logps=None) == _lib.SINK_ATTN_ERR_INVALID_ARG
    for name in ("lse", "g", "gx"):
        assert _logps_bwd(**{name: None}) == _lib.SINK_ATTN_ERR_INVALID_ARG
    assert _logps_bwd(gstride=99) == _lib.SINK_ATTN_ERR_INVALID_ARG
    assert _logps_bwd(gbstride=204) == _lib.SINK_ATTN_ERR_INVALID_ARG
    assert _logps_bwd(gx=FAKE + 4) == _lib.SINK_ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("gbstride,gstride,ok", [
    (208, 104, True),     # batch-major, packed
    (0, 104, False),      # every batch on the same rows
    (200, 104, False),    # batch 1 starts inside batch 0's last row
    (104, 208, True),     # position-major ([seq, batch, vocab] storage)
    (96, 208, False),     # rows of one position overlap
    (104, 200, False),    # position 1 starts inside position 0's last row
])
def test_logps_gradient_rows_must_not_overlap(gbstride, gstride, ok):
    # lse=None stops an accepted layout at the next check, before any launch
    assert _logps_bwd(gbstride=gbstride, gstride=gstride, lse=None) == _lib.SINK_ATTN_ERR_INVALID_ARG
    msg = _lib.load().sink_attn_last_error().decode()
    assert ("overlap" not in msg and "lse" in msg) if ok else ("overlap" in msg)


def test_logps_input_rows_may_overlap():
    # reading is harmless: a zero batch stride (the same rows for every batch) is accepted
    assert _logps_fwd(bstride=0, logps=None) == _lib.SINK_ATTN_ERR_INVALID_ARG  # only logps is missing
    assert "logps" in _lib.load().sink_attn_last_error().decode()


def test_logps_zero_rows_is_a_no_op():
    for b, n in ((0, 4), (4, 0)):
        assert _logps_fwd(batch=b, seq=n, logits=None, ids=None, logps=None) == _lib.SINK_ATTN_OK
        assert _logps_bwd(batch=b, seq=n, logits=None, ids=None, lse=None, g=None, gx=None) == _lib.SINK_ATTN_OK


def _bwd_noalloc(p, **override):
    lib = _lib.load()
    args = dict(q=FAKE, k=FAKE, v=FAKE, sinks=FAKE, o=FAKE, lse=FAKE, dout=FAKE, dq=FAKE,
                dk=FAKE, dv=FAKE, dsinks=FAKE)
    args.update(override)
    ptr = ctypes.byref(p) if p is not None else None
    return lib.sink_attn_bwd_noalloc(ptr, args["q"], args["k"], args["v"], args["sinks"], args["o"],
                                     args["lse"], args["dout"], args["dq"], args["dk"], args["dv"],
                                     args["dsinks"], None)


@pytest.mark.parametrize("name", ["q", "k", "v", "sinks", "o", "lse", "dout", "dq", "dk", "dv",
                                  "dsinks"])
def test_noalloc_bwd_null_tensor(name):
    assert _bwd_noalloc(_good_params(), **{name: None}) == _lib.SINK_ATTN_ERR_INVALID_ARG


def test_noalloc_bwd_bad_params():
    p = _good_params()
    p.head_dim = 12
    assert _bwd_noalloc(p) == _lib.SINK_ATTN_ERR_INVALID_ARG
    assert _bwd_noalloc(None) == _lib.SINK_ATTN_ERR_INVALID_ARG


def test_noalloc_bwd_rejects_workspace_beyond_its_buffer():
    """The row statistics alone (2 floats per query head and token) exceed the
    fixed buffer: rejected with the size it would need, before any HIP call."""
    lib = _lib.load()
    T, hq = 140000, 64
    assert 2 * 4 * hq * T > _lib.SINK_ATTN_NOALLOC_SCRATCH_BYTES
    p = _good_params(T=T, hq=hq, hkv=8)
    assert _bwd_noalloc(p) == _lib.SINK_ATTN_ERR_UNSUPPORTED
    msg = lib.sink_attn_last_error().decode()
    assert "needs" in msg and str(_lib.SINK_ATTN_NOALLOC_SCRATCH_BYTES) in msg


def test_noalloc_bwd_respects_a_fixed_split_that_does_not_fit(monkeypatch):
    """With SINK_ATTN_DKDV_HEADS fixing one head per dK/dV workgroup, the
    float partial sums of 4096 tokens x 64 heads do not fit: rejected rather
    than silently taking another split."""
    monkeypatch.setenv("SINK_ATTN_DKDV_HEADS", "1")
    p = _good_params(T=4096, hq=64, hkv=8)
    assert _bwd_noalloc(p) == _lib.SINK_ATTN_ERR_UNSUPPORTED


def test_noalloc_buffer_size_matches_header():
    text = open(os.path.join(ROOT, "include", "sink_attn.h")).read()
    m = re.search(r"#define SINK_ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.SINK_ATTN_NOALLOC_SCRATCH_BYTES
