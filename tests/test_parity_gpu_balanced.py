"""Balanced decode calls on the GPU vs the CPU oracle, through the C ABI.

A small batch cut into many splits (16 or more) whose whole work is large
runs the balanced build: the device sizes the splits from the batch's total
pages (about 512 workgroups' worth) instead of the longest length alone, the
later splits stay empty, and the merge must skip them.  Each case below is
chosen so that the splits do grow (checked against the sizing rule before
the call), with ragged lengths that include empty, one-token and one-page
sequences, for every pool format and the windowed call.  Attention within
max-abs 2e-3 and relative L2 1e-3 of the oracle's fp64 attention over its own
cache (whose bytes the other parity tests pin bit-exactly)."""
import numpy as np
import pytest
import torch

import bit_kv_cache_block_amd as kvq
import oracle
import workloads
from workloads import bits

pytestmark = pytest.mark.gpu
DEV = "cuda"
MAX_ABS, REL_L2 = 2e-3, 1e-3
PAGE = 16
BALANCE_MAX_BATCH = 32

# twelve ragged sequences of up to 4096 tokens (256 pages) and 1823 pages in all
LENS = [0, 1, 17, 4096, 3000, 4000, 3900, 2500, 4090, 3333, 64, 4095]
# thirty-two sequences of up to 1024 tokens (the largest batch that balances)
LENS32 = [int(x) for x in np.random.default_rng(5).integers(1, 1025, 32)]
LENS32[3], LENS32[9], LENS32[20] = 0, 1024, 16


def setup_module(_):
    oracle.build(force=False)


def _odt(t):
    return oracle.BF16 if t.dtype == torch.bfloat16 else oracle.F16


def assert_close(got, want, label=""):
    err = np.abs(got - want)
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    print(f"[{label}] max-abs {err.max():.3e} rel-L2 {rel:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err.max() <= MAX_ABS, f"{label}: max-abs {err.max():.3e}"
    assert rel <= REL_L2, f"{label}: rel-L2 {rel:.3e}"


def _grown_split(w, splits, ws_bytes, extra_slots=0):
    """(planned pages per split, pages per split of a balanced call) for this
    case, from the planned split count the workspace size reveals and the
    sizing rule the kernels follow; asserts that the call is balanced and that
    its splits grow."""
    nsplit = ws_bytes // (w.batch * w.hq * (w.d + 2) * 4) - extra_slots
    pages_max = (w.max_seq_len + PAGE - 1) // PAGE
    sp = ((pages_max + nsplit - 1) // nsplit + 3) // 4 * 4
    total = int(sum((int(n) + PAGE - 1) // PAGE for n in w.seq_lens))
    want = (total * w.hkv + 511) // 512
    grown = max(sp, (want + 3) // 4 * 4)
    assert nsplit >= 16 and w.batch <= BALANCE_MAX_BATCH, (nsplit, w.batch)
    assert pages_max * w.batch * w.hkv > sp * 512, "the host would not balance this case"
    assert grown > sp, f"S{splits}: splits of {sp} pages would not grow ({grown})"
    return sp, grown


def _stale_ws(nbytes):
    return torch.full((max(nbytes, 16),), 0xFF, dtype=torch.uint8, device=DEV)   # NaN as fp32


def _inputs(w):
    return (w.q.to(DEV), torch.from_numpy(w.block_table).to(DEV), torch.from_numpy(w.seq_lens).to(DEV))


def _check_empty_rows(got, w):
    for b, n in enumerate(w.seq_lens):
        if n == 0:
            assert not got[b].any(), f"empty sequence {b} not zero"


@pytest.mark.parametrize("hq,block", [(8, 64), (32, 64), (64, 0), (128, 64)])
def test_balanced_int4(hq, block):
    """Token-wise INT4, rotated and plain, one to sixteen query heads per KV
    head (all three head-set shapes of the kernel; with one set per
    workgroup the 1536- and 1024-workgroup grids take the 128-VGPR build)."""
    w = workloads.random_decode(41, batch=len(LENS), hq=hq, hkv=8, d=128, block=block, seq_lens=LENS)
    cache = kvq.Int4Cache(w.num_pages, w.hkv, w.d, block, DEV)
    kvq.kvq_append_paged(cache, w.k.to(DEV), w.v.to(DEV), w.slot_mapping.to(DEV))
    pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
    oracle.append_int4(pool, w.num_pages, w.hkv, w.d, block, bits(w.k), bits(w.v), _odt(w.k),
                       w.slot_mapping.numpy())
    want = oracle.decode_int4(pool, w.hkv, w.d, block, bits(w.q), _odt(w.q), w.block_table,
                              w.seq_lens, w.sm_scale)
    q, bt, sl = _inputs(w)
    for splits in (16, 40, 64):
        nb = kvq.kvq_decode_workspace_bytes(w.batch, w.hq, w.hkv, w.d, w.max_seq_len, splits)
        sp, grown = _grown_split(w, splits, nb)
        out = kvq.kvq_decode_attn(cache, q, bt, sl, w.max_seq_len, w.sm_scale, workspace=_stale_ws(nb),
                                  num_splits=splits)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        _check_empty_rows(got, w)
        assert_close(got, want, f"balanced int4 hq{hq} block{block} S{splits} ({sp} -> {grown} pages)")


def test_balanced_int4_batch32_fp16_d64():
    """The largest batch the device balances (its lengths read by 32 of the
    wave's 64 lanes), head_dim 64, fp16 query."""
    w = workloads.random_decode(43, batch=32, hq=32, hkv=8, d=64, block=32, dtype=torch.float16,
                                seq_lens=LENS32)
    cache = kvq.Int4Cache(w.num_pages, w.hkv, w.d, 32, DEV)
    kvq.kvq_append_paged(cache, w.k.to(DEV), w.v.to(DEV), w.slot_mapping.to(DEV))
    pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
    oracle.append_int4(pool, w.num_pages, w.hkv, w.d, 32, bits(w.k), bits(w.v), _odt(w.k),
                       w.slot_mapping.numpy())
    want = oracle.decode_int4(pool, w.hkv, w.d, 32, bits(w.q), _odt(w.q), w.block_table,
                              w.seq_lens, w.sm_scale)
    q, bt, sl = _inputs(w)
    nb = kvq.kvq_decode_workspace_bytes(w.batch, w.hq, w.hkv, w.d, w.max_seq_len, 64)
    sp, grown = _grown_split(w, 64, nb)
    out = kvq.kvq_decode_attn(cache, q, bt, sl, w.max_seq_len, w.sm_scale, workspace=_stale_ws(nb),
                              num_splits=64)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    _check_empty_rows(got, w)
    assert_close(got, want, f"balanced int4 batch 32 d64 ({sp} -> {grown} pages)")


@pytest.mark.parametrize("fmt", ["int8", "int4g32", "int4g64", "mxfp4", "bf16"])
def test_balanced_other_pools(fmt):
    w = workloads.random_decode(47, batch=len(LENS), hq=32, hkv=8, d=128, block=64, seq_lens=LENS)
    k, v, sm = w.k.to(DEV), w.v.to(DEV), w.slot_mapping.to(DEV)
    kb, vb, odt, slots = bits(w.k), bits(w.v), _odt(w.k), w.slot_mapping.numpy()
    qb, oq = bits(w.q), _odt(w.q)
    if fmt == "int8":
        cache = kvq.Int8Cache(w.num_pages, w.hkv, w.d, 64, DEV)
        kvq.kvq_append_paged_int8(cache, k, v, sm)
        pool = oracle.new_int8_pool(w.num_pages, w.hkv, w.d)
        oracle.append_int8(pool, w.num_pages, w.hkv, w.d, 64, kb, vb, odt, slots)
        want = oracle.decode_int8(pool, w.hkv, w.d, 64, qb, oq, w.block_table, w.seq_lens, w.sm_scale)
        fn = kvq.kvq_decode_attn_int8
    elif fmt.startswith("int4g"):
        group = int(fmt[5:])
        cache = kvq.Int4GroupedCache(w.num_pages, w.hkv, w.d, 64, group, DEV)
        kvq.kvq_append_paged_int4g(cache, k, v, sm)
        pool = oracle.new_int4g_pool(w.num_pages, w.hkv, w.d, group)
        oracle.append_int4g(pool, w.num_pages, w.hkv, w.d, 64, group, kb, vb, odt, slots)
        want = oracle.decode_int4g(pool, w.hkv, w.d, 64, group, qb, oq, w.block_table, w.seq_lens,
                                   w.sm_scale)
        fn = kvq.kvq_decode_attn_int4g
    elif fmt == "mxfp4":
        cache = kvq.MxFp4Cache(w.num_pages, w.hkv, w.d, 64, DEV)
        kvq.kvq_append_paged_mxfp4(cache, k, v, sm)
        pool = oracle.new_mxfp4_pool(w.num_pages, w.hkv, w.d)
        oracle.append_mxfp4(pool, w.num_pages, w.hkv, w.d, 64, kb, vb, odt, slots)
        want = oracle.decode_mxfp4(pool, w.hkv, w.d, 64, qb, oq, w.block_table, w.seq_lens, w.sm_scale)
        fn = kvq.kvq_decode_attn_mxfp4
    else:
        cache = kvq.Bf16Cache(w.num_pages, w.hkv, w.d, DEV)
        kvq.kvq_append_paged_bf16(cache, k, v, sm)
        pool = oracle.new_bf16_pool(w.num_pages, w.hkv, w.d)
        oracle.append_bf16(pool, w.num_pages, w.hkv, w.d, kb, vb, odt, slots)
        want = oracle.decode_bf16(pool, w.hkv, w.d, qb, oq, w.block_table, w.seq_lens, w.sm_scale)
        fn = kvq.kvq_decode_attn_bf16
    q, bt, sl = _inputs(w)
    for splits in (16, 64):
        nb = kvq.kvq_decode_workspace_bytes(w.batch, w.hq, w.hkv, w.d, w.max_seq_len, splits)
        sp, grown = _grown_split(w, splits, nb)
        out = fn(cache, q, bt, sl, w.max_seq_len, w.sm_scale, workspace=_stale_ws(nb), num_splits=splits)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        _check_empty_rows(got, w)
        assert_close(got, want, f"balanced {fmt} S{splits} ({sp} -> {grown} pages)")


def test_balanced_windowed():
    """The windowed call's INT4 pass balanced: its merge skips the empty
    splits and still takes the window pass's partial from the last slot."""
    w_sink, w_recent = 4, 124
    w = workloads.random_decode(53, batch=len(LENS), hq=32, hkv=8, d=128, block=64, seq_lens=LENS)
    cache = kvq.Int4Cache(w.num_pages, w.hkv, w.d, 64, DEV)
    kvq.kvq_append_paged(cache, w.k.to(DEV), w.v.to(DEV), w.slot_mapping.to(DEV))
    pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
    oracle.append_int4(pool, w.num_pages, w.hkv, w.d, 64, bits(w.k), bits(w.v), _odt(w.k),
                       w.slot_mapping.numpy())
    rng = np.random.default_rng(21)
    wbt, npages = workloads.window_layout(w.batch, w_sink, w_recent, rng)
    slots = workloads.window_slots(wbt, w.token_seq, w.token_pos, w.seq_lens, w_sink, w_recent)
    win = kvq.Bf16Cache(npages, w.hkv, w.d, DEV)
    kvq.kvq_append_paged_bf16(win, w.k.to(DEV), w.v.to(DEV), torch.from_numpy(slots).to(DEV))
    wpool = oracle.new_bf16_pool(npages, w.hkv, w.d)
    oracle.append_bf16(wpool, npages, w.hkv, w.d, bits(w.k), bits(w.v), _odt(w.k), slots)
    want = oracle.decode_windowed(pool, wpool, w.hkv, w.d, 64, bits(w.q), _odt(w.q), w.block_table, wbt,
                                  w.seq_lens, w_sink, w_recent, w.sm_scale)
    q, bt, sl = _inputs(w)
    for splits in (16, 64):
        nb = kvq.kvq_decode_windowed_workspace_bytes(w.batch, w.hq, w.hkv, w.d, w.max_seq_len, splits)
        sp, grown = _grown_split(w, splits, nb, extra_slots=1)
        out = kvq.kvq_decode_attn_windowed(cache, win, q, bt, torch.from_numpy(wbt).to(DEV), sl,
                                           w.max_seq_len, w_sink, w_recent, w.sm_scale,
                                           workspace=_stale_ws(nb), num_splits=splits)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        _check_empty_rows(got, w)
        assert_close(got, want, f"balanced windowed S{splits} ({sp} -> {grown} pages)")
