"""Block-table entries outside [0, num_pages) inside a sequence's range (a
negative id, an id past the pool): every decode kernel leaves that page's
tokens out of the softmax, as the oracle does (a row whose pages are all
absent is zero).  Pages are bit-exact as appended; attention within the
usual tolerance, with the automatic split plan and with forced splits."""
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


def setup_module(_):
    oracle.build(force=False)


def _close(got, want, label):
    err = np.abs(got - want).max()
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    print(f"[{label}] max-abs {err:.3e} rel-L2 {rel:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err <= MAX_ABS and rel <= REL_L2, label


def _workload():
    w = workloads.random_decode(31, batch=5, hq=8, hkv=2, d=128, block=64,
                                seq_lens=[70, 100, 33, 0, 40])
    bt = w.block_table.copy()
    bt[0][1] = -1                    # a middle page
    bt[1][2] = w.num_pages + 7       # past the pool
    bt[2][:3] = -2                   # every page of the sequence
    bt[4][2] = -1                    # the last, partial page
    return w, bt


# (cache class, append, decode, oracle pool, oracle append, oracle decode, extra args)
KINDS = {
    "int4_b64": (64,), "int4_plain": (0,), "int8": (64,), "int4g64": (64,), "mxfp4": (64,), "bf16": (0,),
}


def _run(kind, w, bt):
    blk = KINDS[kind][0]
    k, v, sm = w.k.to(DEV), w.v.to(DEV), w.slot_mapping.to(DEV)
    kb, vb, smn = bits(w.k), bits(w.v), w.slot_mapping.numpy()
    if kind.startswith("int4_"):
        cache = kvq.Int4Cache(w.num_pages, w.hkv, w.d, blk, DEV)
        kvq.kvq_append_paged(cache, k, v, sm)
        pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
        oracle.append_int4(pool, w.num_pages, w.hkv, w.d, blk, kb, vb, oracle.BF16, smn)
        dec = kvq.kvq_decode_attn
        want = oracle.decode_int4(pool, w.hkv, w.d, blk, bits(w.q), oracle.BF16, bt, w.seq_lens, w.sm_scale)
    elif kind == "int8":
        cache = kvq.Int8Cache(w.num_pages, w.hkv, w.d, blk, DEV)
        kvq.kvq_append_paged_int8(cache, k, v, sm)
        pool = oracle.new_int8_pool(w.num_pages, w.hkv, w.d)
        oracle.append_int8(pool, w.num_pages, w.hkv, w.d, blk, kb, vb, oracle.BF16, smn)
        dec = kvq.kvq_decode_attn_int8
        want = oracle.decode_int8(pool, w.hkv, w.d, blk, bits(w.q), oracle.BF16, bt, w.seq_lens, w.sm_scale)
    elif kind == "int4g64":
        cache = kvq.Int4GroupedCache(w.num_pages, w.hkv, w.d, blk, 64, DEV)
        kvq.kvq_append_paged_int4g(cache, k, v, sm)
        pool = oracle.new_int4g_pool(w.num_pages, w.hkv, w.d, 64)
        oracle.append_int4g(pool, w.num_pages, w.hkv, w.d, blk, 64, kb, vb, oracle.BF16, smn)
        dec = kvq.kvq_decode_attn_int4g
        want = oracle.decode_int4g(pool, w.hkv, w.d, blk, 64, bits(w.q), oracle.BF16, bt, w.seq_lens,
                                   w.sm_scale)
    elif kind == "mxfp4":
        cache = kvq.MxFp4Cache(w.num_pages, w.hkv, w.d, blk, DEV)
        kvq.kvq_append_paged_mxfp4(cache, k, v, sm)
        pool = oracle.new_mxfp4_pool(w.num_pages, w.hkv, w.d)
        oracle.append_mxfp4(pool, w.num_pages, w.hkv, w.d, blk, kb, vb, oracle.BF16, smn)
        dec = kvq.kvq_decode_attn_mxfp4
        want = oracle.decode_mxfp4(pool, w.hkv, w.d, blk, bits(w.q), oracle.BF16, bt, w.seq_lens,
                                   w.sm_scale)
    else:
        cache = kvq.Bf16Cache(w.num_pages, w.hkv, w.d, DEV)
        kvq.kvq_append_paged_bf16(cache, k, v, sm)
        pool = oracle.new_bf16_pool(w.num_pages, w.hkv, w.d)
        oracle.append_bf16(pool, w.num_pages, w.hkv, w.d, kb, vb, oracle.BF16, smn)
        dec = kvq.kvq_decode_attn_bf16
        want = oracle.decode_bf16(pool, w.hkv, w.d, bits(w.q), oracle.BF16, bt, w.seq_lens, w.sm_scale)
    torch.cuda.synchronize()
    assert np.array_equal(cache.pool.cpu().numpy().reshape(-1), pool.reshape(-1)), f"{kind}: pages"
    return cache, dec, want


@pytest.mark.parametrize("kind", list(KINDS))
def test_absent_pages_are_left_out(kind):
    w, bt = _workload()
    cache, dec, want = _run(kind, w, bt)
    assert not want[2].any() and not want[3].any()
    q = w.q.to(DEV)
    btd = torch.from_numpy(bt).to(DEV)
    sl = torch.from_numpy(w.seq_lens).to(DEV)
    for splits in (0, 1, 3):
        out = dec(cache, q, btd, sl, w.max_seq_len, w.sm_scale, num_splits=splits)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert not got[2].any() and not got[3].any(), f"{kind} S{splits}: rows without tokens"
        _close(got, want, f"absent pages {kind} S{splits}")


def test_absent_pages_windowed():
    """The windowed call: absent pages in the INT4 block table and in the
    window table both leave their tokens out, as in the oracle."""
    w_sink, w_recent = 4, 12
    w = workloads.random_decode(33, batch=5, hq=8, hkv=2, d=128, block=64,
                                seq_lens=[70, 100, 9, 0, 40])
    rng = np.random.default_rng(12)
    wbt, npages = workloads.window_layout(w.batch, w_sink, w_recent, rng)
    slots = workloads.window_slots(wbt, w.token_seq, w.token_pos, w.seq_lens, w_sink, w_recent)
    win = kvq.Bf16Cache(npages, w.hkv, w.d, DEV)
    kvq.kvq_append_paged_bf16(win, w.k.to(DEV), w.v.to(DEV), torch.from_numpy(slots).to(DEV))
    wpool = oracle.new_bf16_pool(npages, w.hkv, w.d)
    oracle.append_bf16(wpool, npages, w.hkv, w.d, bits(w.k), bits(w.v), oracle.BF16, slots)
    cache = kvq.Int4Cache(w.num_pages, w.hkv, w.d, 64, DEV)
    kvq.kvq_append_paged(cache, w.k.to(DEV), w.v.to(DEV), w.slot_mapping.to(DEV))
    pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
    oracle.append_int4(pool, w.num_pages, w.hkv, w.d, 64, bits(w.k), bits(w.v), oracle.BF16,
                       w.slot_mapping.numpy())
    bt, wt = w.block_table.copy(), wbt.copy()
    bt[0][1] = -1                    # INT4 tokens 16..31 of sequence 0
    wt[0][0] = npages + 5            # every window token of sequence 0 (past the window pool)
    bt[1][3] = w.num_pages + 7       # INT4 tokens 48..63 of sequence 1
    bt[2][0] = -2                    # sequence 2 lies in its window only, ...
    wt[2][:] = -1                    # ... whose pages are absent too: a zero row
    bt[4][2] = -1                    # the last, partial page of sequence 4: in its recent window
    want = oracle.decode_windowed(pool, wpool, w.hkv, w.d, 64, bits(w.q), oracle.BF16, bt, wt,
                                  w.seq_lens, w_sink, w_recent, w.sm_scale)
    assert not want[2].any() and not want[3].any()
    torch.cuda.synchronize()
    for splits in (0, 1, 3):
        out = kvq.kvq_decode_attn_windowed(cache, win, w.q.to(DEV), torch.from_numpy(bt).to(DEV),
                                           torch.from_numpy(wt).to(DEV),
                                           torch.from_numpy(w.seq_lens).to(DEV), w.max_seq_len,
                                           w_sink, w_recent, w.sm_scale, num_splits=splits)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert not got[2].any() and not got[3].any(), f"windowed S{splits}: rows without tokens"
        _close(got, want, f"absent pages windowed S{splits}")
