"""kvq_decode_attn_noalloc (split-K partials in the library's static device
scratch, for callers that cannot allocate) against kvq_decode_attn with a
caller workspace: the same kernels and split plan, so the outputs must be
identical, and both within the attention tolerance of the oracle.  Two calls
in a row, the second with a smaller input; and a call whose plan needs more
scratch than the library holds is refused before anything is launched."""
import ctypes as C

import numpy as np
import pytest
import torch

import bit_kv_cache_block_amd as kvq
import oracle
import workloads
from workloads import bits

DEV = "cuda"
FAKE = 1 << 20


def test_noalloc_refuses_oversized_plans_on_the_host():
    """Batch 256 of 64 query heads cut into 8 splits needs 68 MB of partials,
    more than the 64 MiB scratch: refused with KVQ_ERR_WORKSPACE_TOO_SMALL
    (no GPU involved; nothing is launched).  The automatic plan of the same
    batch (stream-K partials, two per range) fits."""
    need = kvq.kvq_decode_workspace_bytes(256, 64, 8, 128, 32768, 8)
    assert need > kvq.NOALLOC_SCRATCH_BYTES
    stream_need = 256 * 2 * 64 * (128 + 2) * 4 + 256 * 8   # 2048 ranges x heads, 2 slots each
    assert stream_need <= kvq.NOALLOC_SCRATCH_BYTES
    desc = kvq._QuantDesc(FAKE, 100000, 16, 8, 128, 64)
    L = kvq.lib()
    st = L.kvq_decode_attn_noalloc(C.byref(desc), FAKE, kvq.KVQ_BF16, 64, FAKE, 2048, FAKE, 256, 32768,
                                   0.088, 8, FAKE, None)
    assert st == kvq.KVQ_ERR_WORKSPACE_TOO_SMALL
    assert b"static scratch" in L.kvq_last_error()


def _case(seed, batch, lens, hq=16, d=128, block=64):
    w = workloads.random_decode(seed, batch=batch, hq=hq, hkv=2, d=d, block=block, seq_lens=lens)
    cache = kvq.Int4Cache(w.num_pages, w.hkv, w.d, block, DEV)
    kvq.kvq_append_paged(cache, w.k.to(DEV), w.v.to(DEV), w.slot_mapping.to(DEV))
    pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
    oracle.append_int4(pool, w.num_pages, w.hkv, w.d, block, bits(w.k), bits(w.v), oracle.BF16,
                       w.slot_mapping.numpy())
    want = oracle.decode_int4(pool, w.hkv, w.d, block, bits(w.q), oracle.BF16, w.block_table,
                              w.seq_lens, w.sm_scale)
    return w, cache, want


@pytest.mark.gpu
def test_noalloc_equals_the_workspace_entry_point_twice():
    oracle.build(force=False)
    cases = [(61, 5, [2500, 700, 1, 0, 1900], 6), (62, 2, [300, 45], 3)]   # the second is smaller
    for seed, batch, lens, splits in cases:
        w, cache, want = _case(seed, batch, lens)
        assert kvq.kvq_decode_workspace_bytes(w.batch, w.hq, w.hkv, w.d, w.max_seq_len, splits) > 0
        q = w.q.to(DEV)
        bt = torch.from_numpy(w.block_table).to(DEV)
        sl = torch.from_numpy(w.seq_lens).to(DEV)
        out_na = torch.full((w.batch, w.hq, w.d), float("nan"), dtype=torch.float32, device=DEV)
        torch.cuda.synchronize()
        print(f"noalloc case seed {seed} batch {batch} splits {splits}", flush=True)
        kvq.kvq_decode_attn_noalloc(cache, q, bt, sl, w.max_seq_len, w.sm_scale, out=out_na, num_splits=splits)
        ref = kvq.kvq_decode_attn(cache, q, bt, sl, w.max_seq_len, w.sm_scale, num_splits=splits)
        torch.cuda.synchronize()
        got, ref = out_na.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(got, ref), f"seed {seed}: differs from kvq_decode_attn"
        err = np.abs(got.astype(np.float64) - want)
        rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
        print(f"[noalloc seed {seed}] max-abs {err.max():.3e} rel-L2 {rel:.3e}", flush=True)
        assert err.max() <= 2e-3 and rel <= 1e-3


@pytest.mark.gpu
def test_noalloc_stream_k_plan_twice():
    """The automatic plan of a batch of 256 (sequence, KV head) pairs whose
    longest sequence is cut takes the stream-K mapping: its partials and the
    merge's per-sequence records go to the static scratch in that layout.
    Bit-identical to kvq_decode_attn on two calls in a row, the second with a
    smaller batch (the first call's records stay in the scratch), and within
    the tolerance of the oracle."""
    oracle.build(force=False)
    rng = np.random.default_rng(17)
    for batch in (72, 64):   # the second is smaller
        lens = np.clip(np.round(np.exp(rng.normal(np.log(200.0), 1.0, batch))), 1, 2000).astype(np.int32)
        lens[5] = 0
        lens[9] = 6000
        w = workloads.random_decode(64 + batch, batch=batch, hq=16, hkv=4, d=128, block=64, seq_lens=lens)
        assert batch * w.hkv >= 256 and (w.max_seq_len + 15) // 16 > 256   # the stream-K rule
        cache = kvq.Int4Cache(w.num_pages, w.hkv, w.d, 64, DEV)
        kvq.kvq_append_paged(cache, w.k.to(DEV), w.v.to(DEV), w.slot_mapping.to(DEV))
        pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
        oracle.append_int4(pool, w.num_pages, w.hkv, w.d, 64, bits(w.k), bits(w.v), oracle.BF16,
                           w.slot_mapping.numpy())
        want = oracle.decode_int4(pool, w.hkv, w.d, 64, bits(w.q), oracle.BF16, w.block_table, w.seq_lens,
                                  w.sm_scale)
        q = w.q.to(DEV)
        bt = torch.from_numpy(w.block_table).to(DEV)
        sl = torch.from_numpy(w.seq_lens).to(DEV)
        out_na = torch.full((w.batch, w.hq, w.d), float("nan"), dtype=torch.float32, device=DEV)
        torch.cuda.synchronize()
        print(f"noalloc stream-K batch {batch}", flush=True)
        kvq.kvq_decode_attn_noalloc(cache, q, bt, sl, w.max_seq_len, w.sm_scale, out=out_na)
        ref = kvq.kvq_decode_attn(cache, q, bt, sl, w.max_seq_len, w.sm_scale)
        torch.cuda.synchronize()
        got, ref = out_na.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(got, ref), f"batch {batch}: differs from kvq_decode_attn"
        err = np.abs(got.astype(np.float64) - want)
        rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
        print(f"[noalloc stream-K batch {batch}] max-abs {err.max():.3e} rel-L2 {rel:.3e}", flush=True)
        assert err.max() <= 2e-3 and rel <= 1e-3
