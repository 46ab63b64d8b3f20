"""MXFP4 variant (E2M1 codes, one E8M0 scale per 32 channels) on the GPU vs
the CPU oracle, through the C ABI: codes and scale bytes bit-exact over the
whole pool, attention within max-abs 2e-3 and relative L2 1e-3 of the
oracle's fp64 attention over its own (bit-identical) cache.  Inputs come from
the seeded generators only."""
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


def _odt(t):
    return oracle.BF16 if t.dtype == torch.bfloat16 else oracle.F16


def gpu_cache(w, block, fill=0):
    cache = kvq.MxFp4Cache(w.num_pages, w.hkv, w.d, block, DEV)
    if fill:
        cache.pool.fill_(fill)
    kvq.kvq_append_paged_mxfp4(cache, w.k.to(DEV), w.v.to(DEV), w.slot_mapping.to(DEV))
    torch.cuda.synchronize()
    return cache


def oracle_pool(w, block, sel=None):
    k, v, sm = w.k, w.v, w.slot_mapping
    if sel is not None:
        k, v, sm = k[sel], v[sel], sm[sel]
    pool = oracle.new_mxfp4_pool(w.num_pages, w.hkv, w.d)
    oracle.append_mxfp4(pool, w.num_pages, w.hkv, w.d, block, bits(k), bits(v), _odt(w.k),
                        sm.cpu().numpy())
    return pool


def oracle_attn(pool, w, block, mask=None):
    return oracle.decode_mxfp4(pool, w.hkv, w.d, block, bits(w.q), _odt(w.q), w.block_table,
                               w.seq_lens, w.sm_scale, mask=mask)


def gpu_decode(cache, w, num_splits=0):
    out = kvq.kvq_decode_attn_mxfp4(cache, w.q.to(DEV), torch.from_numpy(w.block_table).to(DEV),
                                    torch.from_numpy(w.seq_lens).to(DEV), w.max_seq_len, w.sm_scale,
                                    num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def assert_close(got, want, label=""):
    err = np.abs(got - want)
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    print(f"[{label}] max-abs {err.max():.3e} rel-L2 {rel:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err.max() <= MAX_ABS, f"{label}: max-abs {err.max():.3e}"
    assert rel <= REL_L2, f"{label}: rel-L2 {rel:.3e}"


def assert_pool_equal(gpu_pool, host_pool, label=""):
    g = gpu_pool.cpu().numpy().reshape(-1)
    diff = np.nonzero(g != host_pool)[0]
    assert diff.size == 0, f"{label}: {diff.size} bytes differ, first at {diff[:8]}"


# ---------------------------------------------------------------- write path

@pytest.mark.parametrize("block", [0, 64])
def test_mxfp4_append_tiny_d64_bitexact(block):
    w = workloads.tiny_decode(1, block=block)
    print(f"mxfp4 append tiny b={block}", flush=True)
    assert_pool_equal(gpu_cache(w, block).pool, oracle_pool(w, block), f"tiny b{block}")


@pytest.mark.parametrize("block", [0, 16, 32, 64, 128])
def test_mxfp4_append_llama_shape_bitexact(block):
    w = workloads.llama8b_decode(2, batch=2, context=1024, block=block)
    print(f"mxfp4 append llama b={block}", flush=True)
    assert_pool_equal(gpu_cache(w, block).pool, oracle_pool(w, block), f"llama b{block}")


def test_mxfp4_append_prefill_student_t_bitexact():
    w = workloads.prefill_append(3, total=8192, nseq=4, lo=512, hi=4096, block=64)
    print("mxfp4 append prefill", flush=True)
    assert_pool_equal(gpu_cache(w, 64).pool, oracle_pool(w, 64), "prefill")


def test_mxfp4_append_ties_saturation_and_degenerate_vectors():
    """Values on the E2M1 midpoints and above 6 after scaling, zero blocks,
    signed zeros, tiny and huge magnitudes, strided input, skipped slots."""
    torch.manual_seed(0)
    t, hkv, d = 37, 3, 128
    wide = torch.randn(t, hkv * d + 64, dtype=torch.float32)
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 6.0, -0.25, -2.5, -5.0])
    wide[4, :12] = mids * 8.0                     # block max 56 -> X = 3: midpoints land exactly
    wide[5, :hkv * d] = 0.0
    wide[6, :hkv * d] = -0.0
    wide[7, :hkv * d] *= 1e-20
    wide[8, :d] = 3.0e4 * torch.sign(wide[8, :d])
    wide[9, 32:64] = 0.0
    wide = wide.to(torch.bfloat16)
    k = wide[:, :hkv * d].view(t, hkv, d)
    v = wide.flip(0)[:, :hkv * d].view(t, hkv, d)
    pages = 5
    slots = np.random.default_rng(1).permutation(pages * 16)[:t].astype(np.int32)
    slots[3] = -1
    slots[10] = pages * 16 + 100
    sm = torch.from_numpy(slots)
    for block in (0, 128):
        print(f"mxfp4 append edge b={block}", flush=True)
        cache = kvq.MxFp4Cache(pages, hkv, d, block, DEV)
        kvq.kvq_append_paged_mxfp4(cache, k.to(DEV), v.to(DEV), sm.to(DEV))
        torch.cuda.synchronize()
        pool = oracle.new_mxfp4_pool(pages, hkv, d)
        oracle.append_mxfp4(pool, pages, hkv, d, block, bits(k.contiguous()), bits(v.contiguous()),
                            oracle.BF16, slots)
        assert_pool_equal(cache.pool, pool, f"edge b{block}")


# ---------------------------------------------------------------- read path

@pytest.mark.parametrize("block,dtype", [(0, torch.float16), (64, torch.bfloat16)])
def test_mxfp4_decode_small(block, dtype):
    w = workloads.random_decode(21, batch=4, hq=8, hkv=2, d=128, block=block, dtype=dtype,
                                seq_lens=[256, 77, 300, 16])
    cache = gpu_cache(w, block)
    want = oracle_attn(oracle_pool(w, block), w, block)
    for splits in (0, 1, 2, 4):
        assert_close(gpu_decode(cache, w, splits), want, f"mxfp4 small b{block} S{splits}")


@pytest.mark.parametrize("block", [0, 64, 128])
def test_mxfp4_decode_llama_shape(block):
    w = workloads.llama8b_decode(2, batch=3, context=4096, block=block)
    cache = gpu_cache(w, block)
    want = oracle_attn(oracle_pool(w, block), w, block)
    assert_close(gpu_decode(cache, w), want, f"mxfp4 llama b{block}")


def test_mxfp4_decode_edge_lengths_over_stale_bytes():
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 100, 300]
    w = workloads.random_decode(11, batch=len(lens), hq=8, hkv=2, d=128, block=64,
                                dtype=torch.bfloat16, seq_lens=lens)
    cache = gpu_cache(w, 64, fill=0xFF)
    want = oracle_attn(oracle_pool(w, 64), w, 64)
    for splits in (0, 1, 2, 3, 100):
        got = gpu_decode(cache, w, splits)
        assert not got[0].any()
        assert_close(got, want, f"mxfp4 edges S{splits}")


@pytest.mark.parametrize("hq,hkv", [(2, 2), (16, 1), (64, 8), (24, 4)])
def test_mxfp4_decode_group_sizes(hq, hkv):
    w = workloads.random_decode(12, batch=3, hq=hq, hkv=hkv, d=128, block=64,
                                seq_lens=[33, 200, 77])
    cache = gpu_cache(w, 64)
    want = oracle_attn(oracle_pool(w, 64), w, 64)
    assert_close(gpu_decode(cache, w), want, f"mxfp4 G{hq // hkv}")


def test_mxfp4_decode_long_context_scaled_channels():
    w = workloads.long_context_decode(4, batch=2, context=16384, block=64)
    cache = gpu_cache(w, 64)
    want = oracle_attn(oracle_pool(w, 64), w, 64)
    for splits in (0, 7):
        assert_close(gpu_decode(cache, w, splits), want, f"mxfp4 long S{splits}")


def test_mxfp4_full_size_llama_layer_sampled():
    """64 x 4096 tokens, block 64, in the benchmark's launch configuration:
    sampled sequences' pages bit-exact, their attention within tolerance."""
    w = workloads.llama8b_decode(2, device=DEV, batch=64, context=4096, block=64)
    cache = kvq.MxFp4Cache(w.num_pages, w.hkv, w.d, 64, DEV)
    kvq.kvq_append_paged_mxfp4(cache, w.k, w.v, w.slot_mapping)
    out = kvq.kvq_decode_attn_mxfp4(cache, w.q, torch.from_numpy(w.block_table).to(DEV),
                                    torch.from_numpy(w.seq_lens).to(DEV), w.max_seq_len, w.sm_scale)
    torch.cuda.synchronize()
    sample = [0, 17, 63]
    sel = torch.from_numpy(np.isin(w.token_seq, sample)).to(DEV)
    pool = oracle_pool(w, 64, sel=sel)
    slab = w.hkv * oracle.mxfp4_slab_bytes(16, w.d)
    gpool = cache.pool.cpu().numpy()
    for b in sample:
        for pg in w.block_table[b][w.block_table[b] >= 0]:
            assert np.array_equal(gpool[pg], pool[int(pg) * slab:(int(pg) + 1) * slab]), f"page {pg}"
    mask = np.zeros((w.batch, w.hq), np.uint8)
    mask[sample] = 1
    want = oracle_attn(pool, w, 64, mask=mask)
    assert_close(out.cpu().numpy().astype(np.float64)[sample], want[sample], "mxfp4 full llama sampled")


@pytest.mark.parametrize("block", [32, 128])
def test_mxfp4_decode_forced_splits_every_block(block):
    """Split partials of a rotated MXFP4 pool, each rotated back before the
    merge: forced splits at blocks 32 and 128 against the oracle."""
    w = workloads.random_decode(91, batch=3, hq=16, hkv=2, d=128, block=block, seq_lens=[700, 300, 1000])
    cache = gpu_cache(w, block)
    want = oracle_attn(oracle_pool(w, block), w, block)
    for splits in (2, 5):
        assert_close(gpu_decode(cache, w, splits), want, f"mxfp4 b{block} S{splits}")


def _crafted_block(rng, X):
    """32 values of one MXFP4 block with shared exponent X (the largest is
    7.5 * 2^X): every tie between E2M1 values, values next to the ties,
    saturating ones, tiny ones that round to zero, both signs."""
    t = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.0, 0.5, 1.0, 1.5, 3.0, 4.0, 6.0, 0.125,
                  0.0625, 0.0, 2.25, 2.75, 0.875, 1.125, 5.5, 4.5, 0.375, 0.625, 3.25, 3.75, 6.25, 0.1875,
                  0.03125], np.float64)
    sign = np.where(rng.random(t.size) < 0.5, -1.0, 1.0)
    vals = np.concatenate([[7.5], sign * t])
    rng.shuffle(vals)
    return vals * 2.0 ** X


@pytest.mark.parametrize("xs", [(-6, 0, 5, 12), (-123, -124, -125, -3), (0, 0, 0, 0)])
def test_mxfp4_append_crafted_ties_bitexact(xs):
    """Crafted blocks through the append (no rotation, so the values reach
    the quantizer as written): every E2M1 tie of both signs, saturation,
    values that round to zero (stored +0), and shared exponents on both sides
    of -124 (subnormal elements at -125), bit-exact against the oracle's
    pool."""
    rng = np.random.default_rng(sum(abs(x) for x in xs) + 7)
    tokens, hkv, d = 48, 2, 128
    k = np.empty((tokens, hkv, d)); v = np.empty((tokens, hkv, d))
    for t in range(tokens):
        for h in range(hkv):
            for blk in range(4):
                X = xs[(blk + t + h) % 4]
                k[t, h, 32 * blk:32 * blk + 32] = _crafted_block(rng, X)
                v[t, h, 32 * blk:32 * blk + 32] = _crafted_block(rng, xs[(blk + 2 * t + h) % 4])
    kb = torch.from_numpy(k).to(torch.bfloat16)
    vb = torch.from_numpy(v).to(torch.bfloat16)
    assert torch.equal(kb.to(torch.float64), torch.from_numpy(k)), "crafted values are bf16-exact"
    w = workloads.random_decode(93, batch=3, hq=8, hkv=hkv, d=d, block=0, seq_lens=[16, 17, 15])
    sm = w.slot_mapping
    cache = kvq.MxFp4Cache(w.num_pages, hkv, d, 0, DEV)
    kvq.kvq_append_paged_mxfp4(cache, kb.to(DEV), vb.to(DEV), sm.to(DEV))
    torch.cuda.synchronize()
    pool = oracle.new_mxfp4_pool(w.num_pages, hkv, d)
    oracle.append_mxfp4(pool, w.num_pages, hkv, d, 0, bits(kb), bits(vb), oracle.BF16, sm.cpu().numpy())
    print(f"mxfp4 crafted {xs}", flush=True)
    assert_pool_equal(cache.pool, pool, f"crafted {xs}")
