"""Token-wise INT8 variant on the GPU vs the CPU oracle, through the C ABI:
codes and fp16 sidecars bit-exact over the whole pool, attention within
max-abs 2e-3 and relative L2 1e-3 of the oracle's fp64 attention over its own
(bit-identical) cache.  Inputs come from the seeded generators only."""
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


def gpu_int8_cache(w, block, fill=0):
    cache = kvq.Int8Cache(w.num_pages, w.hkv, w.d, block, DEV)
    if fill:
        cache.pool.fill_(fill)
    kvq.kvq_append_paged_int8(cache, w.k.to(DEV), w.v.to(DEV), w.slot_mapping.to(DEV))
    torch.cuda.synchronize()
    return cache


def oracle_int8_pool(w, block, sel=None):
    k, v, sm = w.k, w.v, w.slot_mapping
    if sel is not None:
        k, v, sm = k[sel], v[sel], sm[sel]
    pool = oracle.new_int8_pool(w.num_pages, w.hkv, w.d)
    oracle.append_int8(pool, w.num_pages, w.hkv, w.d, block, bits(k), bits(v), _odt(w.k),
                       sm.cpu().numpy())
    return pool


def oracle_attn(pool, w, block, mask=None):
    return oracle.decode_int8(pool, w.hkv, w.d, block, bits(w.q), _odt(w.q), w.block_table,
                              w.seq_lens, w.sm_scale, mask=mask)


def gpu_decode(cache, w, num_splits=0):
    out = kvq.kvq_decode_attn_int8(cache, w.q.to(DEV), torch.from_numpy(w.block_table).to(DEV),
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
def test_int8_append_tiny_fp16_bitexact(block):
    w = workloads.tiny_decode(1, block=block)
    print(f"int8 append tiny block={block}", flush=True)
    assert_pool_equal(gpu_int8_cache(w, block).pool, oracle_int8_pool(w, block), f"tiny b{block}")


@pytest.mark.parametrize("block", [0, 16, 32, 64, 128])
def test_int8_append_llama_shape_bitexact(block):
    w = workloads.llama8b_decode(2, batch=2, context=1024, block=block)
    print(f"int8 append llama b={block}", flush=True)
    assert_pool_equal(gpu_int8_cache(w, block).pool, oracle_int8_pool(w, block), f"llama b{block}")


def test_int8_append_prefill_student_t_bitexact():
    w = workloads.prefill_append(3, total=8192, nseq=4, lo=512, hi=4096, block=64)
    print("int8 append prefill", flush=True)
    assert_pool_equal(gpu_int8_cache(w, 64).pool, oracle_int8_pool(w, 64), "prefill")


def test_int8_append_strided_tokens_skip_slots_and_degenerate_vectors():
    torch.manual_seed(0)
    t, hkv, d = 37, 3, 128
    wide = torch.randn(t, hkv * d + 64, dtype=torch.float32)
    wide[5, :hkv * d] = 0.75                    # constant
    wide[6, :hkv * d] = -0.0                    # signed zeros
    wide[7, :hkv * d] *= 1e-7                   # subnormal scale
    wide[8, :d] = 3.0e4 * torch.sign(wide[8, :d])
    wide = wide.to(torch.bfloat16)
    k = wide[:, :hkv * d].view(t, hkv, d)
    v = wide.flip(0)[:, :hkv * d].view(t, hkv, d)
    pages = 5
    slots = np.random.default_rng(1).permutation(pages * 16)[:t].astype(np.int32)
    slots[3] = -1
    slots[9] = pages * 16 + 100
    sm = torch.from_numpy(slots)
    for block in (0, 32, 128):
        print(f"int8 append edge b={block}", flush=True)
        cache = kvq.Int8Cache(pages, hkv, d, block, DEV)
        kvq.kvq_append_paged_int8(cache, k.to(DEV), v.to(DEV), sm.to(DEV))
        torch.cuda.synchronize()
        pool = oracle.new_int8_pool(pages, hkv, d)
        oracle.append_int8(pool, pages, hkv, d, block, bits(k.contiguous()), bits(v.contiguous()),
                           oracle.BF16, slots)
        assert_pool_equal(cache.pool, pool, f"edge b{block}")


# ---------------------------------------------------------------- read path

@pytest.mark.parametrize("block", [0, 64])
def test_int8_decode_tiny(block):
    w = workloads.tiny_decode(1, block=block)
    cache = gpu_int8_cache(w, block)
    want = oracle_attn(oracle_int8_pool(w, block), w, block)
    for splits in (0, 1, 2, 4):
        assert_close(gpu_decode(cache, w, splits), want, f"int8 tiny b{block} S{splits}")


@pytest.mark.parametrize("block", [0, 64, 128])
def test_int8_decode_llama_shape(block):
    w = workloads.llama8b_decode(2, batch=3, context=4096, block=block)
    cache = gpu_int8_cache(w, block)
    want = oracle_attn(oracle_int8_pool(w, block), w, block)
    assert_close(gpu_decode(cache, w), want, f"int8 llama b{block}")


@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.float16)])
def test_int8_decode_edge_lengths_over_stale_bytes(d, dtype):
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 100, 300]
    w = workloads.random_decode(11, batch=len(lens), hq=8, hkv=2, d=d, block=d // 2, dtype=dtype,
                                seq_lens=lens)
    cache = gpu_int8_cache(w, w.block, fill=0xFF)
    want = oracle_attn(oracle_int8_pool(w, w.block), w, w.block)
    for splits in (0, 1, 2, 3, 100):
        got = gpu_decode(cache, w, splits)
        assert not got[0].any()
        assert_close(got, want, f"int8 edges d{d} S{splits}")


@pytest.mark.parametrize("hq,hkv,d", [(2, 2, 128), (4, 2, 64), (16, 1, 128), (64, 8, 128), (32, 4, 64)])
def test_int8_decode_group_sizes(hq, hkv, d):
    w = workloads.random_decode(12, batch=3, hq=hq, hkv=hkv, d=d, block=64,
                                seq_lens=[33, 200, 77])
    cache = gpu_int8_cache(w, 64)
    want = oracle_attn(oracle_int8_pool(w, 64), w, 64)
    assert_close(gpu_decode(cache, w), want, f"int8 G{hq // hkv} d{d}")


def test_int8_decode_long_context_scaled_channels():
    w = workloads.long_context_decode(4, batch=2, context=16384, block=64)
    cache = gpu_int8_cache(w, 64)
    want = oracle_attn(oracle_int8_pool(w, 64), w, 64)
    for splits in (0, 7):
        assert_close(gpu_decode(cache, w, splits), want, f"int8 long S{splits}")


def test_int8_full_size_llama_layer_sampled():
    """64 x 4096 tokens, block 64, in the benchmark's launch configuration:
    sampled sequences' pages bit-exact, their attention within tolerance."""
    w = workloads.llama8b_decode(2, device=DEV, batch=64, context=4096, block=64)
    cache = kvq.Int8Cache(w.num_pages, w.hkv, w.d, 64, DEV)
    kvq.kvq_append_paged_int8(cache, w.k, w.v, w.slot_mapping)
    out = kvq.kvq_decode_attn_int8(cache, w.q, torch.from_numpy(w.block_table).to(DEV),
                                   torch.from_numpy(w.seq_lens).to(DEV), w.max_seq_len, w.sm_scale)
    torch.cuda.synchronize()
    sample = [0, 41, 63]
    sel = torch.from_numpy(np.isin(w.token_seq, sample)).to(DEV)
    pool = oracle_int8_pool(w, 64, sel=sel)
    slab = w.hkv * oracle.int8_slab_bytes(16, w.d)
    gpool = cache.pool.cpu().numpy()
    for b in sample:
        for pg in w.block_table[b][w.block_table[b] >= 0]:
            assert np.array_equal(gpool[pg], pool[int(pg) * slab:(int(pg) + 1) * slab]), f"page {pg}"
    mask = np.zeros((w.batch, w.hq), np.uint8)
    mask[sample] = 1
    want = oracle_attn(pool, w, 64, mask=mask)
    assert_close(out.cpu().numpy().astype(np.float64)[sample], want[sample], "int8 full llama sampled")
