"""C-ABI checks that need no GPU: the library loads, exports every function
include/kvq.h declares, and host-side validation rejects bad arguments before
anything is launched (only invalid calls are made here, so no HIP work is
ever enqueued)."""
import ctypes as C
import os
import re

import pytest

import bit_kv_cache_block_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20          # an aligned, never-dereferenced address


def _header_functions():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _header_functions()
    assert len(names) == 24
    assert sorted(kvq.EXPORTED) == names
    L = kvq.lib()
    for name in names:
        assert hasattr(L, name), name


def test_abi_version_and_status_strings():
    L = kvq.lib()
    assert L.kvq_abi_version() == 1
    assert L.kvq_status_string(3) == b"KVQ_ERR_WORKSPACE_TOO_SMALL"
    assert L.kvq_status_string(99) == b"KVQ_ERR_UNKNOWN"


def test_page_bytes():
    assert kvq.kvq_int4_page_bytes(16, 8, 128) == 8 * 2176
    assert kvq.kvq_int4_page_bytes(16, 2, 64) == 2 * 1152
    assert kvq.kvq_bf16_page_bytes(16, 8, 128) == 8 * 8192
    assert kvq.kvq_int8_page_bytes(16, 8, 128) == 8 * 4224
    assert kvq.kvq_int8_page_bytes(16, 2, 64) == 2 * 2176
    assert kvq.kvq_int4g_page_bytes(16, 8, 128, 64) == 8 * 16 * (128 + 16)
    assert kvq.kvq_int4g_page_bytes(16, 8, 128, 32) == 8 * 16 * (128 + 32)
    assert kvq.kvq_int4g_page_bytes(16, 8, 128, 48) == 0
    assert kvq.kvq_mxfp4_page_bytes(16, 8, 128) == 8 * 2176
    assert kvq.kvq_mxfp4_page_bytes(16, 2, 64) == 2 * 16 * 68


def _int4(num_pages=64, page=16, hkv=2, d=64, block=64, pool=FAKE):
    return kvq._QuantDesc(pool, num_pages, page, hkv, d, block)


def _append(desc, k=FAKE, v=FAKE, dtype=kvq.KVQ_BF16, stride=128, slots=FAKE, n=4, fn="kvq_append_paged"):
    L = kvq.lib()
    return getattr(L, fn)(C.byref(desc) if desc is not None else None, k, v, dtype, stride,
                          slots, n, None)


@pytest.mark.parametrize("desc,kw,status", [
    (None, {}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    (_int4(d=96), {}, kvq.KVQ_ERR_UNSUPPORTED),
    (_int4(page=32), {}, kvq.KVQ_ERR_UNSUPPORTED),
    (_int4(block=8), {}, kvq.KVQ_ERR_UNSUPPORTED),
    (_int4(block=128, d=64), {}, kvq.KVQ_ERR_UNSUPPORTED),
    (_int4(num_pages=0), {}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    (_int4(pool=0), {}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    (_int4(pool=FAKE + 4), {}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    (_int4(), {"k": 0}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    (_int4(), {"slots": 0}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    (_int4(), {"k": FAKE + 8}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    (_int4(), {"stride": 64}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    (_int4(), {"stride": 132}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    (_int4(), {"stride": (1 << 24) + 8}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    (_int4(), {"dtype": 7}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    (_int4(), {"n": -1}, kvq.KVQ_ERR_INVALID_ARGUMENT),
])
@pytest.mark.parametrize("fn", ["kvq_append_paged", "kvq_append_paged_int8"])
def test_append_validation(desc, kw, status, fn):
    assert _append(desc, fn=fn, **kw) == status
    assert kvq.lib().kvq_last_error() != b""


def test_append_zero_tokens_is_a_noop():
    assert _append(_int4(), k=0, v=0, slots=0, n=0) == kvq.KVQ_OK
    assert _append(_int4(), k=0, v=0, slots=0, n=0, fn="kvq_append_paged_int8") == kvq.KVQ_OK


def _decode(desc, q=FAKE, dtype=kvq.KVQ_BF16, hq=8, bt=FAKE, maxp=256, sl=FAKE, batch=4,
            maxlen=4096, sm=0.125, splits=0, out=FAKE, ws=FAKE, wsb=0, fn="kvq_decode_attn"):
    # the defaults need a split-K workspace (4 x 4096 tokens over 2 KV heads),
    # so with wsb = 0 every call here is rejected before anything is launched
    L = kvq.lib()
    return getattr(L, fn)(C.byref(desc), q, dtype, hq, bt, maxp, sl, batch, maxlen, sm, splits,
                          out, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    ({"hq": 7}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    ({"hq": 64}, kvq.KVQ_ERR_UNSUPPORTED),           # group 32 > 16
    ({"q": 0}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    ({"out": FAKE + 4}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    ({"bt": 0}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    ({"maxp": 8}, kvq.KVQ_ERR_INVALID_ARGUMENT),      # 8 pages < 4096 tokens
    ({"sm": float("nan")}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    ({"batch": -1}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    ({"splits": -2}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    ({"wsb": 0}, kvq.KVQ_ERR_WORKSPACE_TOO_SMALL),
])
@pytest.mark.parametrize("fn", ["kvq_decode_attn", "kvq_decode_attn_int8"])
def test_decode_validation(kw, status, fn):
    assert _decode(_int4(), fn=fn, **kw) == status


@pytest.mark.parametrize("fn", ["kvq_decode_attn", "kvq_decode_attn_int8"])
def test_decode_rejects_bad_block(fn):
    assert _decode(_int4(block=8), fn=fn, wsb=1 << 30) == kvq.KVQ_ERR_UNSUPPORTED
    assert _decode(_int4(d=96), fn=fn, wsb=1 << 30) == kvq.KVQ_ERR_UNSUPPORTED


def test_decode_workspace_too_small_by_one():
    need = kvq.kvq_decode_workspace_bytes(4, 8, 2, 64, 4096, 0)
    assert need > 0
    assert _decode(_int4(), wsb=need - 1) == kvq.KVQ_ERR_WORKSPACE_TOO_SMALL
    assert _decode(_int4(), wsb=need - 1, fn="kvq_decode_attn_int8") == kvq.KVQ_ERR_WORKSPACE_TOO_SMALL


def _grouped(group=64, d=128, block=64):
    return kvq._GroupedDesc(FAKE, 64, 16, 2, d, block, group)


@pytest.mark.parametrize("desc,status", [
    (_grouped(group=16), kvq.KVQ_ERR_UNSUPPORTED),
    (_grouped(group=128), kvq.KVQ_ERR_UNSUPPORTED),
    (_grouped(group=64, d=64, block=128), kvq.KVQ_ERR_UNSUPPORTED),
    (_grouped(group=0), kvq.KVQ_ERR_UNSUPPORTED),
])
def test_grouped_entry_points_validate(desc, status):
    L = kvq.lib()
    assert L.kvq_append_paged_int4g(C.byref(desc), FAKE, FAKE, 1, 256, FAKE, 4, None) == status
    assert L.kvq_decode_attn_int4g(C.byref(desc), FAKE, 1, 8, FAKE, 256, FAKE, 4, 4096, 0.1, 0,
                                   FAKE, FAKE, 1 << 30, None) == status
    ok = _grouped()
    assert L.kvq_append_paged_int4g(C.byref(ok), FAKE, FAKE, 1, 64, FAKE, 4, None) == kvq.KVQ_ERR_INVALID_ARGUMENT
    assert L.kvq_decode_attn_int4g(C.byref(ok), FAKE, 1, 8, FAKE, 256, FAKE, 4, 4096, 0.1, 0,
                                   FAKE, FAKE, 0, None) == kvq.KVQ_ERR_WORKSPACE_TOO_SMALL


def test_mxfp4_entry_points_validate():
    L = kvq.lib()
    d64 = kvq._QuantDesc(FAKE, 64, 16, 2, 64, 64)
    assert L.kvq_decode_attn_mxfp4(C.byref(d64), FAKE, 1, 8, FAKE, 256, FAKE, 4, 4096, 0.1, 0,
                                   FAKE, FAKE, 1 << 30, None) == kvq.KVQ_ERR_UNSUPPORTED
    bad = kvq._QuantDesc(FAKE, 64, 16, 2, 128, 8)
    assert L.kvq_append_paged_mxfp4(C.byref(bad), FAKE, FAKE, 1, 256, FAKE, 4, None) == kvq.KVQ_ERR_UNSUPPORTED
    ok = kvq._QuantDesc(FAKE, 64, 16, 2, 128, 64)
    assert L.kvq_append_paged_mxfp4(C.byref(ok), FAKE, FAKE, 1, 128, FAKE, 4, None) == kvq.KVQ_ERR_INVALID_ARGUMENT
    assert L.kvq_decode_attn_mxfp4(C.byref(ok), FAKE, 1, 8, FAKE, 256, FAKE, 4, 4096, 0.1, 0,
                                   FAKE, FAKE, 0, None) == kvq.KVQ_ERR_WORKSPACE_TOO_SMALL
    assert L.kvq_append_paged_mxfp4(C.byref(ok), 0, 0, 1, 256, 0, 0, None) == kvq.KVQ_OK


def test_binding_keeps_int4_and_int8_pools_apart():
    c8 = kvq.Int8Cache(2, 2, 64, 64, device="cpu")
    c4 = kvq.Int4Cache(2, 2, 64, 64, device="cpu")
    assert c8.pool.shape[1] == kvq.kvq_int8_page_bytes(16, 2, 64)
    assert c4.pool.shape[1] == kvq.kvq_int4_page_bytes(16, 2, 64)
    with pytest.raises(TypeError):
        kvq.kvq_append_paged(c8, None, None, None)
    with pytest.raises(TypeError):
        kvq.kvq_decode_attn_int8(c4, None, None, None, 0)
    cg = kvq.Int4GroupedCache(2, 2, 128, 64, 32, device="cpu")
    assert cg.pool.shape[1] == kvq.kvq_int4g_page_bytes(16, 2, 128, 32)
    with pytest.raises(TypeError):
        kvq.kvq_decode_attn(cg, None, None, None, 0)
    cm = kvq.MxFp4Cache(2, 2, 128, 64, device="cpu")
    assert cm.pool.shape[1] == kvq.kvq_mxfp4_page_bytes(16, 2, 128)
    with pytest.raises(TypeError):
        kvq.kvq_append_paged(cm, None, None, None)


def test_decode_zero_batch_is_a_noop():
    assert _decode(_int4(), batch=0, q=0, bt=0, sl=0, out=0) == kvq.KVQ_OK


def test_bf16_entry_points_validate():
    L = kvq.lib()
    bad = kvq._Bf16Desc(FAKE, 4, 16, 2, 100)
    assert L.kvq_append_paged_bf16(C.byref(bad), FAKE, FAKE, 1, 128, FAKE, 1, None) == kvq.KVQ_ERR_UNSUPPORTED
    ok = kvq._Bf16Desc(FAKE, 4, 16, 2, 64)
    assert kvq.kvq_decode_workspace_bytes(4, 8, 2, 64, 4096, 0) > 0
    assert L.kvq_decode_attn_bf16(C.byref(ok), FAKE, 1, 8, FAKE, 256, FAKE, 4, 4096, 0.1, 0, FAKE,
                                  FAKE, 0, None) == kvq.KVQ_ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("batch,hkv,maxlen,stream", [(64, 8, 4096, False), (8, 8, 131072, False),
                                                      (256, 8, 32768, True), (32, 8, 32768, True),
                                                      (16, 8, 32768, False), (1, 8, 32768, False),
                                                      (4, 2, 256, False), (3, 1, 1, False)])
def test_workspace_covers_every_split(batch, hkv, maxlen, stream):
    """With a split count given, the workspace holds (D + 2) floats per
    (sequence, head, split), and the split plan covers the longest sequence
    with splits of whole 4-page steps.  With the automatic plan of a batch of
    at least 256 (sequence, KV head) pairs whose longest sequence is cut, it
    also holds the stream-K partials: (D + 2) floats for two slots per range
    and query head of the largest grid (2048 workgroups, whole KV heads) and
    two int32 per sequence."""
    hq, d = hkv * 4, 128
    ws = kvq.kvq_decode_workspace_bytes(batch, hq, hkv, d, maxlen, 0)
    sk = -(-2048 // hkv) * hkv * 2 * (hq // hkv) * (d + 2) * 4 + batch * 8
    if stream:
        assert ws >= sk
    if ws != sk:   # the planned splits (of a decode with no stream-K build) need more
        assert ws % (batch * hq * (d + 2) * 4) == 0
        nsplit = ws // (batch * hq * (d + 2) * 4)
        pages = (maxlen + 15) // 16
        assert (1 if ws else 0) <= nsplit <= max(1, (pages + 3) // 4)
    for s in (1, 2, 5):
        ws_s = kvq.kvq_decode_workspace_bytes(batch, hq, hkv, d, maxlen, s)
        assert ws_s // (batch * hq * (d + 2) * 4) <= s
    assert kvq.kvq_decode_workspace_bytes(batch, hq, hkv, d, maxlen, 1) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kvq, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(kvq, "_lib_handle", None)
    with pytest.raises(RuntimeError, match="libkvq.so not found"):
        kvq.kvq_int4_page_bytes(16, 8, 128)


def _windowed(desc, win, ws_bytes=0, w_sink=4, w_recent=12, wmaxp=1, maxlen=4096, wt=FAKE):
    L = kvq.lib()
    return L.kvq_decode_attn_windowed(C.byref(desc), C.byref(win), FAKE, kvq.KVQ_BF16, 8, FAKE, 256, wt,
                                      wmaxp, FAKE, 4, maxlen, w_sink, w_recent, 0.125, 0, FAKE, FAKE,
                                      ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    ({"w_sink": -1}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    ({"w_recent": -3}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    ({"wmaxp": 0}, kvq.KVQ_ERR_INVALID_ARGUMENT),        # 0 pages < 16 window tokens
    ({"wt": 0}, kvq.KVQ_ERR_INVALID_ARGUMENT),
    ({"ws_bytes": 0}, kvq.KVQ_ERR_WORKSPACE_TOO_SMALL),
])
def test_windowed_decode_validation(kw, status):
    assert _windowed(_int4(), kvq._Bf16Desc(FAKE, 4, 16, 2, 64), **kw) == status


def test_windowed_decode_rejects_mismatched_window_pool():
    assert _windowed(_int4(), kvq._Bf16Desc(FAKE, 4, 16, 4, 64)) == kvq.KVQ_ERR_INVALID_ARGUMENT
    assert _windowed(_int4(), kvq._Bf16Desc(FAKE, 4, 16, 2, 128)) == kvq.KVQ_ERR_INVALID_ARGUMENT


def test_windowed_workspace_holds_a_partial_per_split_and_the_window():
    """The INT4 pass always stores partials and the window pass stores one
    more per row (the split merge finishes the call), so even one split needs
    two slots; split counts match kvq_decode_attn's plan (a batch this small
    takes no stream-K mapping)."""
    row = 4 * 8 * (64 + 2) * 4
    for maxlen in (16, 4096, 131072):
        for s in (0, 2, 5):
            plain = kvq.kvq_decode_workspace_bytes(4, 8, 2, 64, maxlen, s)
            win = kvq.kvq_decode_windowed_workspace_bytes(4, 8, 2, 64, maxlen, s)
            assert win == (plain if plain else row) + row


# ---------------------------------------------------------------- binding checks
# The Python binding checks shapes and devices before it hands anything to the
# library; every call below raises ValueError on the host, so nothing is
# launched (all tensors are host tensors and no GPU is needed).

def _host_decode_args(batch=3, hq=8, hkv=2, d=64, pages=4):
    import torch
    cache = kvq.Int4Cache(16, hkv, d, 64, device="cpu")
    q = torch.zeros((batch, hq, d), dtype=torch.bfloat16)
    bt = torch.zeros((batch, pages), dtype=torch.int32)
    sl = torch.full((batch,), 16, dtype=torch.int32)
    return cache, q, bt, sl


@pytest.mark.parametrize("fault,match", [
    ("short_table", "block_table must be"),
    ("flat_table", "block_table must be"),
    ("short_lens", "seq_lens must hold"),
    ("bad_out", "out must be"),
    ("host_pool", "cache pool must be a GPU tensor"),
])
def test_binding_decode_rejects_bad_shapes_and_devices(fault, match):
    import torch
    cache, q, bt, sl = _host_decode_args()
    out = None
    if fault == "short_table":
        bt = bt[:2].contiguous()
    elif fault == "flat_table":
        bt = bt.reshape(-1).contiguous()
    elif fault == "short_lens":
        sl = sl[:2].contiguous()
    elif fault == "bad_out":
        out = torch.zeros((3, 8, 32), dtype=torch.float32)
    with pytest.raises(ValueError, match=match):
        kvq.kvq_decode_attn(cache, q, bt, sl, 64, out=out)
    with pytest.raises(ValueError, match=match):
        kvq.kvq_decode_attn_bf16(kvq.Bf16Cache(16, 2, 64, device="cpu"), q, bt, sl, 64, out=out)


def test_binding_windowed_rejects_bad_window_table():
    import torch
    cache, q, bt, sl = _host_decode_args()
    win = kvq.Bf16Cache(8, 2, 64, device="cpu")
    with pytest.raises(ValueError, match="window_table must be"):
        kvq.kvq_decode_attn_windowed(cache, win, q, bt, torch.zeros((2, 1), dtype=torch.int32), sl,
                                     64, 4, 12)
    with pytest.raises(ValueError, match="cache pool must be a GPU tensor"):
        kvq.kvq_decode_attn_windowed(cache, win, q, bt, torch.zeros((3, 1), dtype=torch.int32), sl,
                                     64, 4, 12)


@pytest.mark.parametrize("fn,cache_fn", [
    ("kvq_append_paged", lambda: kvq.Int4Cache(4, 2, 64, 64, device="cpu")),
    ("kvq_append_paged_int8", lambda: kvq.Int8Cache(4, 2, 64, 64, device="cpu")),
    ("kvq_append_paged_bf16", lambda: kvq.Bf16Cache(4, 2, 64, device="cpu")),
])
def test_binding_append_rejects_bad_slots_and_devices(fn, cache_fn):
    import torch
    k = torch.zeros((5, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="slot_mapping has 4 entries for 5 tokens"):
        getattr(kvq, fn)(cache_fn(), k, k.clone(), torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="cache pool must be a GPU tensor"):
        getattr(kvq, fn)(cache_fn(), k, k.clone(), torch.zeros(5, dtype=torch.int32))
