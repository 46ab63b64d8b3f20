"""The stream-K mapping of the plain INT4-family decodes on the GPU vs the CPU
oracle, through the C ABI.  The automatic plan takes it for a batch of at
least 256 (sequence, KV head) pairs whose longest sequence the plan would cut
(here: max_seq_len above 4096, so at least two 256-page splits): the batch's
pages, one sequence after another (each also counted as a fixed cost), are
cut per KV head into ranges, one workgroup each (equal ranges for a small
run; for a large one, longer ranges for the workgroups dispatched first on
each CU), and a sequence met by several ranges is merged from their
partials.  Ragged lognormal batches with empty sequences, single-token
sequences, absent pages and one sequence spanning many ranges; GQA 4, 8 and
16 (one, two and four sets of heads), head_dim 64 and 128, token-wise INT4
(rotated and not), INT8 and grouped INT4.  Pools bit-exact as appended;
attention within max-abs 2e-3 and relative L2 1e-3 of the oracle's fp64
attention over its own cache.  Inputs come from the seeded generators only."""
import math

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


def _lengths(seed, batch, long_len):
    """Lognormal lengths (median 200 tokens) with edge cases planted: an
    empty sequence, single-token ones, a page-aligned one and one long
    sequence that crosses many ranges."""
    rng = np.random.default_rng(seed)
    lens = np.clip(np.round(np.exp(rng.normal(math.log(200.0), 1.0, batch))), 1, 3000).astype(np.int32)
    lens[3] = 0
    lens[5] = 1
    lens[-1] = 1
    lens[9] = 256
    lens[11] = long_len
    return lens


def _streamed(batch, hkv, maxlen):
    # the rule the library applies with num_splits = 0
    return batch * hkv >= 256 and (maxlen + 15) // 16 > 256


def _run(kind, w, bt):
    blk = w.block
    k, v, sm = w.k.to(DEV), w.v.to(DEV), w.slot_mapping.to(DEV)
    kb, vb, smn = bits(w.k), bits(w.v), w.slot_mapping.numpy()
    qb = bits(w.q)
    if kind == "int4":
        cache = kvq.Int4Cache(w.num_pages, w.hkv, w.d, blk, DEV)
        kvq.kvq_append_paged(cache, k, v, sm)
        pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
        oracle.append_int4(pool, w.num_pages, w.hkv, w.d, blk, kb, vb, oracle.BF16, smn)
        dec = kvq.kvq_decode_attn
        want = oracle.decode_int4(pool, w.hkv, w.d, blk, qb, oracle.BF16, bt, w.seq_lens, w.sm_scale)
    elif kind == "int8":
        cache = kvq.Int8Cache(w.num_pages, w.hkv, w.d, blk, DEV)
        kvq.kvq_append_paged_int8(cache, k, v, sm)
        pool = oracle.new_int8_pool(w.num_pages, w.hkv, w.d)
        oracle.append_int8(pool, w.num_pages, w.hkv, w.d, blk, kb, vb, oracle.BF16, smn)
        dec = kvq.kvq_decode_attn_int8
        want = oracle.decode_int8(pool, w.hkv, w.d, blk, qb, oracle.BF16, bt, w.seq_lens, w.sm_scale)
    else:
        gs = int(kind[5:])
        cache = kvq.Int4GroupedCache(w.num_pages, w.hkv, w.d, blk, gs, DEV)
        kvq.kvq_append_paged_int4g(cache, k, v, sm)
        pool = oracle.new_int4g_pool(w.num_pages, w.hkv, w.d, gs)
        oracle.append_int4g(pool, w.num_pages, w.hkv, w.d, blk, gs, kb, vb, oracle.BF16, smn)
        dec = kvq.kvq_decode_attn_int4g
        want = oracle.decode_int4g(pool, w.hkv, w.d, blk, gs, qb, oracle.BF16, bt, w.seq_lens, w.sm_scale)
    torch.cuda.synchronize()
    assert np.array_equal(cache.pool.cpu().numpy().reshape(-1), pool.reshape(-1)), f"{kind}: pages"
    return cache, dec, want


def _decode(dec, cache, w, bt, num_splits=0):
    out = dec(cache, w.q.to(DEV), torch.from_numpy(bt).to(DEV), torch.from_numpy(w.seq_lens).to(DEV),
              w.max_seq_len, w.sm_scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


# (kind, batch, hq, hkv, head_dim, block, long sequence)
CASES = [
    ("int4", 64, 32, 4, 128, 64, 9000),     # two sets of heads (GQA 8)
    ("int4", 64, 32, 4, 128, 0, 5000),      # unrotated
    ("int4", 64, 16, 4, 128, 128, 7000),    # one set (GQA 4)
    ("int4", 128, 32, 2, 128, 64, 6000),    # four sets (GQA 16)
    ("int4", 64, 32, 4, 64, 32, 8000),      # head_dim 64
    ("int8", 64, 32, 4, 128, 64, 6000),
    ("int4g64", 64, 16, 4, 128, 64, 6000),
    ("int4g32", 64, 32, 4, 128, 32, 5000),
]


@pytest.mark.parametrize("kind,batch,hq,hkv,d,block,long_len", CASES)
def test_stream_ragged_batch(kind, batch, hq, hkv, d, block, long_len):
    lens = _lengths(100 + batch + hq + d + block, batch, long_len)
    w = workloads.random_decode(61, batch=batch, hq=hq, hkv=hkv, d=d, block=block, seq_lens=lens)
    assert _streamed(batch, hkv, w.max_seq_len)
    print(f"stream {kind} B{batch} hq{hq} hkv{hkv} d{d} b{block} max {w.max_seq_len}", flush=True)
    bt = w.block_table.copy()
    bt[0][0] = -1                     # absent pages: first, middle, past the pool
    bt[11][40] = -3
    bt[11][41] = w.num_pages + 5
    bt[12][:] = -1                    # every page of a sequence absent
    cache, dec, want = _run(kind, w, bt)
    got = _decode(dec, cache, w, bt)
    assert not got[3].any() and not want[3].any()    # empty sequence: zero rows
    _close(got, want, f"stream {kind} B{batch} hq{hq} d{d} b{block}")
    # the same cache with forced splits (the planned mapping) agrees too
    _close(_decode(dec, cache, w, bt, num_splits=5), want, f"planned {kind} S5")


def test_stream_one_sequence_across_every_range():
    """All sequences a single token but one of 60000 tokens: that one is met
    by every range of its KV head and merged from all their partials."""
    batch = 64
    lens = np.ones(batch, np.int32)
    lens[17] = 60000
    w = workloads.random_decode(62, batch=batch, hq=32, hkv=4, d=128, block=64, seq_lens=lens)
    assert _streamed(batch, 4, w.max_seq_len)
    print("stream one long sequence", flush=True)
    cache, dec, want = _run("int4", w, w.block_table)
    _close(_decode(dec, cache, w, w.block_table), want, "stream one long")


def test_stream_all_sequences_empty():
    """Every length zero with a bound that would be cut: no range has pages,
    every row is zero (the merge writes them)."""
    batch = 64
    w = workloads.random_decode(63, batch=batch, hq=32, hkv=4, d=128, block=64,
                                seq_lens=np.full(batch, 20, np.int32))
    cache, dec, _ = _run("int4", w, w.block_table)
    zero = np.zeros(batch, np.int32)
    bt = np.full((batch, 8192 // 16), -1, np.int32)   # rows long enough for the bound
    bt[:, :w.block_table.shape[1]] = w.block_table
    out = torch.full((batch, 32, 128), 7.0, dtype=torch.float32, device=DEV)
    kvq.kvq_decode_attn(cache, w.q.to(DEV), torch.from_numpy(bt).to(DEV),
                        torch.from_numpy(zero).to(DEV), 8192, w.sm_scale, out=out)
    torch.cuda.synchronize()
    assert _streamed(batch, 4, 8192)
    assert not out.cpu().numpy().any()


def test_stream_repeated_calls_are_identical():
    """The merge's records and partials live in the workspace and are written
    anew by each call: two calls on one workspace with different lengths give
    each call's own result, and a call repeated gives the same bits."""
    batch = 64
    lens_a = _lengths(7, batch, 6000)
    w = workloads.random_decode(64, batch=batch, hq=32, hkv=4, d=128, block=64, seq_lens=lens_a)
    cache, dec, want = _run("int4", w, w.block_table)
    ws = torch.empty(kvq.kvq_decode_workspace_bytes(batch, 32, 4, 128, w.max_seq_len), dtype=torch.uint8,
                     device=DEV)
    q, bt = w.q.to(DEV), torch.from_numpy(w.block_table).to(DEV)
    lens_b = lens_a.copy()
    lens_b[11] = 4500                 # the long sequence shorter: other ranges, other records
    lens_b[3] = 50
    outs = []
    for lens in (lens_a, lens_b, lens_a):
        outs.append(kvq.kvq_decode_attn(cache, q, bt, torch.from_numpy(lens).to(DEV), w.max_seq_len, w.sm_scale,
                                        workspace=ws).cpu().numpy())
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[2])
    _close(outs[0].astype(np.float64), want, "stream call 1")
    pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
    oracle.append_int4(pool, w.num_pages, w.hkv, w.d, 64, bits(w.k), bits(w.v), oracle.BF16,
                       w.slot_mapping.numpy())
    want_b = oracle.decode_int4(pool, w.hkv, w.d, 64, bits(w.q), oracle.BF16, w.block_table, lens_b, w.sm_scale)
    _close(outs[1].astype(np.float64), want_b, "stream call 2")


@pytest.mark.parametrize("seed", list(range(8)))
def test_stream_random_ragged_batches(seed):
    """Seeded random batches that take the stream-K mapping: 64 to 160
    sequences over 4 KV heads, GQA 4 or 8, rotated or not, lognormal lengths
    with zeros, single tokens and one sequence past 4096 tokens, and a few
    absent pages; range ends then fall at many places relative to sequence
    and page boundaries."""
    rng = np.random.default_rng(1000 + seed)
    batch = int(rng.integers(64, 161))
    hq = int(rng.choice([16, 32]))
    block = int(rng.choice([0, 64]))
    lens = np.clip(np.round(np.exp(rng.normal(math.log(150.0), 1.2, batch))), 0, 2500).astype(np.int32)
    lens[rng.integers(0, batch, 3)] = 0
    lens[rng.integers(0, batch, 3)] = 1
    lens[int(rng.integers(0, batch))] = int(rng.integers(4200, 9000))
    w = workloads.random_decode(70 + seed, batch=batch, hq=hq, hkv=4, d=128, block=block, seq_lens=lens)
    assert _streamed(batch, 4, w.max_seq_len)
    print(f"stream random seed {seed}: B{batch} hq{hq} b{block} max {w.max_seq_len} "
          f"tokens {int(lens.sum())}", flush=True)
    bt = w.block_table.copy()
    for _ in range(4):   # absent pages inside some sequences' ranges
        b = int(rng.integers(0, batch))
        npg = (int(lens[b]) + 15) // 16
        if npg:
            bt[b][int(rng.integers(0, npg))] = -1 if rng.random() < 0.5 else w.num_pages + 3
    cache, dec, want = _run("int4", w, bt)
    _close(_decode(dec, cache, w, bt), want, f"stream random seed {seed}")


def _sampled_oracle(w, bt, rows):
    """The oracle's pool and attention for the sequences in `rows` only: their
    tokens appended from host copies, their rows of the block table decoded."""
    cum = np.concatenate([[0], np.cumsum(w.seq_lens.astype(np.int64))])
    toks = np.concatenate([np.arange(cum[b], cum[b + 1]) for b in rows]).astype(np.int64)
    sel = torch.from_numpy(toks)
    k, v = w.k.index_select(0, sel.to(w.k.device)).cpu(), w.v.index_select(0, sel.to(w.v.device)).cpu()
    sm = w.slot_mapping.cpu().numpy()[toks]
    pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
    oracle.append_int4(pool, w.num_pages, w.hkv, w.d, w.block, bits(k), bits(v), oracle.BF16, sm)
    q = w.q.cpu()[torch.from_numpy(np.asarray(rows))]
    want = oracle.decode_int4(pool, w.hkv, w.d, w.block, bits(q), oracle.BF16, np.ascontiguousarray(bt[rows]),
                              np.ascontiguousarray(w.seq_lens[rows]), w.sm_scale)
    return pool, want


@pytest.mark.parametrize("hq,block", [(32, 64), (16, 128)])
def test_stream_weighted_ranges_large_batch(hq, block):
    """A batch large enough (at least 64 units of the run per range whatever
    the device's occupancy: over 32768 pages per KV head) that the stream-K
    cut gives each dispatch slot its own range length, with a sequence that
    spans many ranges, an empty one and single-token ones.  Pages of the
    sampled sequences bit-exact against the oracle's, their attention within
    tolerance of the oracle's."""
    batch, hkv = 104, 4
    rng = np.random.default_rng(4242 + hq)
    lens = np.clip(np.round(np.exp(rng.normal(math.log(5000.0), 0.6, batch))), 1, 20000).astype(np.int32)
    lens[3] = 0
    lens[5] = 1
    lens[8] = 1
    lens[40] = 60000
    assert int(((lens + 15) // 16).sum()) > 32768
    w = workloads.random_decode(80 + hq, device=DEV, batch=batch, hq=hq, hkv=hkv, d=128, block=block, seq_lens=lens)
    assert _streamed(batch, hkv, w.max_seq_len)
    print(f"stream weighted hq{hq} b{block}: tokens {int(lens.sum())} pages {int(((lens + 15) // 16).sum())}",
          flush=True)
    cache = kvq.Int4Cache(w.num_pages, hkv, 128, block, DEV)
    kvq.kvq_append_paged(cache, w.k, w.v, w.slot_mapping)
    bt = w.block_table
    got = _decode(kvq.kvq_decode_attn, cache, w, bt)
    assert np.isfinite(got).all() and not got[3].any()
    rows = [3, 5, 8, 40] + [int(x) for x in rng.choice([b for b in range(batch) if b not in (3, 5, 8, 40)], 5,
                                                       replace=False)]
    pool, want = _sampled_oracle(w, bt, rows)
    gpu_pool = cache.pool.cpu().numpy().reshape(w.num_pages, -1)
    ora_pool = pool.reshape(w.num_pages, -1)
    for b in rows:
        pages = bt[b][: (int(lens[b]) + 15) // 16]
        assert np.array_equal(gpu_pool[pages], ora_pool[pages]), f"pages of sequence {b}"
    _close(got[rows], want, f"stream weighted hq{hq} b{block}")
