"""GPU path vs the CPU oracle, through the C ABI.

Codes and fp16 sidecars: bit-exact over the whole pool.  Attention: within
max-abs 2e-3 and relative L2 1e-3 of the oracle's fp64 attention over its own
(bit-identical) cache.  Every input comes from the seeded generators; nothing
the oracle sees comes from the GPU."""
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


def gpu_int4_cache(w, block, k=None, v=None):
    cache = kvq.Int4Cache(w.num_pages, w.hkv, w.d, block, DEV)
    k = w.k if k is None else k
    v = w.v if v is None else v
    kvq.kvq_append_paged(cache, k.to(DEV), v.to(DEV), w.slot_mapping.to(DEV))
    torch.cuda.synchronize()
    return cache


def oracle_int4_pool(w, block, sel=None):
    k, v, sm = w.k, w.v, w.slot_mapping
    if sel is not None:
        k, v, sm = k[sel], v[sel], sm[sel]
    pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
    oracle.append_int4(pool, w.num_pages, w.hkv, w.d, block, bits(k), bits(v), _odt(w.k),
                       sm.cpu().numpy())
    return pool


def gpu_decode(cache, w, num_splits=0, bf16=False):
    fn = kvq.kvq_decode_attn_bf16 if bf16 else kvq.kvq_decode_attn
    out = fn(cache, w.q.to(DEV), torch.from_numpy(w.block_table).to(DEV),
             torch.from_numpy(w.seq_lens).to(DEV), w.max_seq_len, w.sm_scale, num_splits=num_splits)
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

@pytest.mark.parametrize("block", [0, 16, 32, 64])
def test_append_tiny_fp16_bitexact(block):
    w = workloads.tiny_decode(1, block=block)
    print(f"append tiny block={block}", flush=True)
    assert_pool_equal(gpu_int4_cache(w, block).pool, oracle_int4_pool(w, block), f"tiny b{block}")


@pytest.mark.parametrize("block", [0, 16, 32, 64, 128])
def test_append_llama_shape_bitexact(block):
    w = workloads.llama8b_decode(2, batch=2, context=1024, block=block)
    print(f"append llama b={block}", flush=True)
    assert_pool_equal(gpu_int4_cache(w, block).pool, oracle_int4_pool(w, block), f"llama b{block}")


@pytest.mark.parametrize("block", [0, 64])
def test_append_prefill_student_t_bitexact(block):
    w = workloads.prefill_append(3, total=8192, nseq=4, lo=512, hi=4096, block=block)
    print(f"append prefill b={block}", flush=True)
    assert_pool_equal(gpu_int4_cache(w, block).pool, oracle_int4_pool(w, block), f"prefill b{block}")


def test_append_strided_tokens_skip_slots_and_degenerate_vectors():
    """Token stride wider than Hkv*D (a view into a fused projection), slot -1,
    constant rows (scale 0), tiny rows (subnormal fp16 scale), a ragged tail."""
    torch.manual_seed(0)
    t, hkv, d = 37, 3, 128
    wide = torch.randn(t, hkv * d + 64, dtype=torch.float32)
    wide[5, :hkv * d] = 0.75                    # constant
    wide[6, :hkv * d] = -0.0                    # signed zeros
    wide[7, :hkv * d] *= 1e-7                   # subnormal scale
    wide[8, :d] = 3.0e4 * torch.sign(wide[8, :d])   # large magnitudes
    wide = wide.to(torch.bfloat16)
    k = wide[:, :hkv * d].view(t, hkv, d)
    v = wide.flip(0)[:, :hkv * d].view(t, hkv, d)
    assert k.stride(0) == hkv * d + 64
    pages = 5
    rng = np.random.default_rng(1)
    slots = rng.permutation(pages * 16)[:t].astype(np.int32)
    slots[3] = -1
    slots[9] = pages * 16 + 100                 # outside the pool: skipped
    sm = torch.from_numpy(slots)
    for block in (0, 32, 128):
        cache = kvq.Int4Cache(pages, hkv, d, block, DEV)
        kvq.kvq_append_paged(cache, k.to(DEV), v.to(DEV), sm.to(DEV))
        torch.cuda.synchronize()
        pool = oracle.new_int4_pool(pages, hkv, d)
        oracle.append_int4(pool, pages, hkv, d, block, bits(k.contiguous()), bits(v.contiguous()),
                           oracle.BF16, slots)
        assert_pool_equal(cache.pool, pool, f"edge b{block}")


@pytest.mark.parametrize("bits_", [4, 8])
@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.float16)])
def test_append_few_token_and_tile_kernels_bitexact(d, dtype, bits_):
    """Appends of at most 1024 tokens take the few-token kernel (a vector over
    D/8 lanes), larger ones the tile kernel: both match the oracle bit for
    bit, on strided rows with constant, signed-zero, tiny and large vectors,
    skipped and out-of-pool slots, for every block size."""
    torch.manual_seed(3)
    hkv = 2
    t_all = 1100
    wide = torch.randn(t_all, hkv * d + 32, dtype=torch.float32)
    wide[5, :hkv * d] = 0.75
    wide[6, :hkv * d] = -0.0
    wide[7, :hkv * d] *= 1e-7
    wide[8, :d] = 3.0e4 * torch.sign(wide[8, :d])
    wide[9, d:2 * d] = 1e-30
    wide = wide.to(dtype)
    k = wide[:, :hkv * d].view(t_all, hkv, d)
    v = wide.flip(0)[:, :hkv * d].view(t_all, hkv, d)
    pages = (t_all + 15) // 16 + 8
    rng = np.random.default_rng(4)
    slots = rng.permutation(pages * 16)[:t_all].astype(np.int32)
    slots[3] = -1
    slots[11] = pages * 16 + 5
    odt = oracle.BF16 if dtype == torch.bfloat16 else oracle.F16
    cls = kvq.Int4Cache if bits_ == 4 else kvq.Int8Cache
    app = kvq.kvq_append_paged if bits_ == 4 else kvq.kvq_append_paged_int8
    new_pool = oracle.new_int4_pool if bits_ == 4 else oracle.new_int8_pool
    oapp = oracle.append_int4 if bits_ == 4 else oracle.append_int8
    for block in [b for b in (0, 16, 32, 64, 128) if b <= d]:
        for t in (1, 7, 1024, t_all):   # t <= 1024: few-token kernel
            cache = cls(pages, hkv, d, block, DEV)
            app(cache, k[:t].to(DEV), v[:t].to(DEV), torch.from_numpy(slots[:t]).to(DEV))
            torch.cuda.synchronize()
            pool = new_pool(pages, hkv, d)
            oapp(pool, pages, hkv, d, block, bits(k[:t].contiguous()), bits(v[:t].contiguous()), odt,
                 slots[:t])
            assert_pool_equal(cache.pool, pool, f"int{bits_} d{d} b{block} t{t}")


def _tie_rows(rng, t, hkv, d, block, levels):
    """Rows whose rotated values y sit on exact ties of the quantizer: y holds
    integers lo + 2j over [lo, lo + 2 levels] with both ends in every group of
    32 channels, so the fp16 scale is 2, the zero lo, and (y - lo) / 2 is an
    integer or an integer plus one half (the odd offsets, about half of them).
    The input is x = H y / sqrt(b) per block (H the Sylvester Hadamard matrix,
    symmetric with H H = b I, so the block transform of x gives back y); at
    b = 16 and 64 every x and every partial sum of the butterfly is a short
    binary fraction, exact in fp16 and fp32."""
    lo = rng.choice([0, -8, -15, 3], size=(t, hkv, 1)).astype(np.float64)
    y = lo + 2.0 * rng.integers(0, levels + 1, size=(t, hkv, d)) - rng.integers(0, 2, size=(t, hkv, d))
    y = np.clip(y, lo, lo + 2 * levels)
    g = y.reshape(t, hkv, d // 32, 32)
    g[..., 0] = lo
    g[..., 17] = lo + 2 * levels
    y = g.reshape(t, hkv, d)
    x = y
    if block > 0:
        h = np.array([[1.0]])
        while h.shape[0] < block:
            h = np.block([[h, h], [h, -h]])
        x = (y.reshape(t, hkv, d // block, block) @ h / np.sqrt(block)).reshape(t, hkv, d)
    xh = x.astype(np.float16)
    assert np.array_equal(xh.astype(np.float64), x), "crafted rows not exact in fp16"
    return torch.from_numpy(xh), y


@pytest.mark.parametrize("kind,block", [("int4", 0), ("int4", 16), ("int4", 64), ("int8", 0),
                                        ("int4g", 0), ("int4g", 64)])
def test_append_exact_ties_bitexact(kind, block):
    """Codes that are exact ties k + 1/2 round to the even neighbour in both
    append kernels (few-token and tile) as in the oracle, for the token-wise
    INT4 and INT8 and the grouped INT4 pools, plain and rotated."""
    rng = np.random.default_rng(11)
    hkv, d, t_all = 2, 128, 1100
    levels = 255 if kind == "int8" else 15
    k, yk = _tie_rows(rng, t_all, hkv, d, block, levels)
    v, _ = _tie_rows(rng, t_all, hkv, d, block, levels)
    ties = (yk - yk.min(axis=2, keepdims=True)) % 2 == 1   # odd offsets from lo
    assert ties.mean() > 0.3
    if block > 0:   # the oracle's rotation gives back y exactly
        for row, want in zip(k[:4].numpy().astype(np.float32).reshape(-1, d), yk[:4].reshape(-1, d)):
            assert np.array_equal(oracle.rotate(row, block).astype(np.float64), want)
    pages = (t_all + 15) // 16 + 4
    slots = rng.permutation(pages * 16)[:t_all].astype(np.int32)
    for t in (9, t_all):   # t <= 1024: few-token kernel
        if kind == "int4":
            cache = kvq.Int4Cache(pages, hkv, d, block, DEV)
            kvq.kvq_append_paged(cache, k[:t].to(DEV), v[:t].to(DEV), torch.from_numpy(slots[:t]).to(DEV))
            pool = oracle.new_int4_pool(pages, hkv, d)
            oracle.append_int4(pool, pages, hkv, d, block, bits(k[:t]), bits(v[:t]), oracle.F16, slots[:t])
        elif kind == "int8":
            cache = kvq.Int8Cache(pages, hkv, d, block, DEV)
            kvq.kvq_append_paged_int8(cache, k[:t].to(DEV), v[:t].to(DEV), torch.from_numpy(slots[:t]).to(DEV))
            pool = oracle.new_int8_pool(pages, hkv, d)
            oracle.append_int8(pool, pages, hkv, d, block, bits(k[:t]), bits(v[:t]), oracle.F16, slots[:t])
        else:
            cache = kvq.Int4GroupedCache(pages, hkv, d, block, 32, DEV)
            kvq.kvq_append_paged_int4g(cache, k[:t].to(DEV), v[:t].to(DEV), torch.from_numpy(slots[:t]).to(DEV))
            pool = oracle.new_int4g_pool(pages, hkv, d, 32)
            oracle.append_int4g(pool, pages, hkv, d, block, 32, bits(k[:t]), bits(v[:t]), oracle.F16,
                                slots[:t])
        torch.cuda.synchronize()
        print(f"ties {kind} b{block} t{t}", flush=True)
        assert_pool_equal(cache.pool, pool, f"ties {kind} b{block} t{t}")


def test_append_bf16_cache_matches_oracle():
    for w in (workloads.tiny_decode(1, block=0), workloads.llama8b_decode(2, batch=2, context=256)):
        cache = kvq.Bf16Cache(w.num_pages, w.hkv, w.d, DEV)
        kvq.kvq_append_paged_bf16(cache, w.k.to(DEV), w.v.to(DEV), w.slot_mapping.to(DEV))
        torch.cuda.synchronize()
        pool = oracle.new_bf16_pool(w.num_pages, w.hkv, w.d)
        oracle.append_bf16(pool, w.num_pages, w.hkv, w.d, bits(w.k), bits(w.v), _odt(w.k),
                           w.slot_mapping.numpy())
        assert_pool_equal(cache.pool, pool, w.name)


# ---------------------------------------------------------------- read path

@pytest.mark.parametrize("block", [0, 64])
def test_decode_tiny(block):
    w = workloads.tiny_decode(1, block=block)
    cache = gpu_int4_cache(w, block)
    pool = oracle_int4_pool(w, block)
    want = oracle.decode_int4(pool, w.hkv, w.d, block, bits(w.q), oracle.F16, w.block_table,
                              w.seq_lens, w.sm_scale)
    for splits in (0, 1, 2, 4):
        assert_close(gpu_decode(cache, w, splits), want, f"tiny b{block} S{splits}")


@pytest.mark.parametrize("d,block", [(128, 16), (128, 32), (128, 64), (128, 128), (64, 16), (64, 32), (64, 64)])
def test_decode_forced_splits_every_block(d, block):
    """Split partials of a rotated pool, each rotated back before the merge
    combines them: every block size, two and five splits, GQA 4 and 8,
    against the oracle."""
    for hq in (8, 16):
        w = workloads.random_decode(90 + block, batch=3, hq=hq, hkv=2, d=d, block=block, seq_lens=[700, 300, 1000])
        cache = gpu_int4_cache(w, block)
        pool = oracle_int4_pool(w, block)
        want = oracle.decode_int4(pool, w.hkv, w.d, block, bits(w.q), _odt(w.q), w.block_table,
                                  w.seq_lens, w.sm_scale)
        for splits in (2, 5):
            assert_close(gpu_decode(cache, w, splits), want, f"splits d{d} b{block} hq{hq} S{splits}")


@pytest.mark.parametrize("block", [0, 16, 32, 64, 128])
def test_decode_llama_shape(block):
    w = workloads.llama8b_decode(2, batch=3, context=4096, block=block)
    cache = gpu_int4_cache(w, block)
    pool = oracle_int4_pool(w, block)
    want = oracle.decode_int4(pool, w.hkv, w.d, block, bits(w.q), oracle.BF16, w.block_table,
                              w.seq_lens, w.sm_scale)
    assert_close(gpu_decode(cache, w), want, f"llama b{block}")


def test_decode_long_context_scaled_channels():
    w = workloads.long_context_decode(4, batch=2, context=16384, block=64)
    cache = gpu_int4_cache(w, 64)
    pool = oracle_int4_pool(w, 64)
    want = oracle.decode_int4(pool, w.hkv, w.d, 64, bits(w.q), oracle.BF16, w.block_table,
                              w.seq_lens, w.sm_scale)
    for splits in (0, 1, 7):
        assert_close(gpu_decode(cache, w, splits), want, f"long S{splits}")


def test_decode_ragged_group8_with_appended_token():
    """70B-shaped layer (GQA 8): fill, append one token per sequence, decode."""
    fill, steps = workloads.concurrency_step(5, batch=8, block=64, steps=1, cap=4096)
    step = steps[0]
    cache = gpu_int4_cache(fill, 64)
    kvq.kvq_append_paged(cache, step.k.to(DEV), step.v.to(DEV), step.slot_mapping.to(DEV))
    pool = oracle_int4_pool(fill, 64)
    oracle.append_int4(pool, step.num_pages, step.hkv, step.d, 64, bits(step.k), bits(step.v),
                       oracle.BF16, step.slot_mapping.numpy())
    assert_pool_equal(cache.pool, pool, "concurrency pool")
    want = oracle.decode_int4(pool, step.hkv, step.d, 64, bits(step.q), oracle.BF16,
                              step.block_table, step.seq_lens, step.sm_scale)
    assert_close(gpu_decode(cache, step), want, "concurrency")


@pytest.mark.parametrize("hq", [8, 16])
@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.float16)])
def test_decode_edge_lengths(d, dtype, hq):
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 100, 300]
    w = workloads.random_decode(11, batch=len(lens), hq=hq, hkv=2, d=d, block=d // 2, dtype=dtype,
                                seq_lens=lens)
    cache = gpu_int4_cache(w, w.block)
    pool = oracle_int4_pool(w, w.block)
    want = oracle.decode_int4(pool, w.hkv, w.d, w.block, bits(w.q), _odt(w.q), w.block_table,
                              w.seq_lens, w.sm_scale)
    for splits in (0, 1, 2, 3, 100):
        got = gpu_decode(cache, w, splits)
        assert not got[0].any()                     # empty sequence -> zeros
        assert_close(got, want, f"edges d{d} hq{hq} S{splits}")


@pytest.mark.parametrize("block", [64, 0])
def test_decode_gqa8_large_grid(block):
    """GQA 8 with more than 4096 workgroups (64 ragged sequences, 8 KV heads,
    10 splits of 8 pages: 5120), the grid size at which the two-set kernel runs its build
    held to three waves per SIMD (one step buffer)."""
    lens = [int(x) for x in np.random.default_rng(3).integers(1, 1200, 64)]
    lens[5], lens[17], lens[40] = 0, 1199, 16
    w = workloads.random_decode(61, batch=64, hq=64, hkv=8, d=128, block=block, seq_lens=lens)
    cache = gpu_int4_cache(w, block)
    pool = oracle_int4_pool(w, block)
    want = oracle.decode_int4(pool, w.hkv, w.d, block, bits(w.q), _odt(w.q), w.block_table,
                              w.seq_lens, w.sm_scale)
    nb = kvq.kvq_decode_workspace_bytes(w.batch, w.hq, w.hkv, w.d, w.max_seq_len, 10)
    assert nb // (w.batch * w.hq * (w.d + 2) * 4) * w.hkv * w.batch > 4096
    got = gpu_decode(cache, w, 10)
    assert not got[5].any()
    assert_close(got, want, f"gqa8 large grid block{block}")


@pytest.mark.parametrize("hq", [4, 8])
@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.float16)])
def test_decode_many_splits_stale_workspace(d, dtype, hq):
    """Few rows cut into many splits (the merge then deals a row's splits to
    several lane groups), with a workspace pre-filled with 0xFF bytes (NaN as
    fp32): slots no split of a short sequence wrote must not leak in."""
    lens = [0, 1, 40, 1000, 4000, 9000]
    w = workloads.random_decode(17, batch=len(lens), hq=hq, hkv=1, d=d, block=d // 2, dtype=dtype,
                                seq_lens=lens)
    cache = gpu_int4_cache(w, w.block)
    pool = oracle_int4_pool(w, w.block)
    want = oracle.decode_int4(pool, w.hkv, w.d, w.block, bits(w.q), _odt(w.q), w.block_table,
                              w.seq_lens, w.sm_scale)
    q = w.q.to(DEV)
    bt = torch.from_numpy(w.block_table).to(DEV)
    sl = torch.from_numpy(w.seq_lens).to(DEV)
    for splits in (4, 9, 17, 33, 64, 140):
        nb = kvq.kvq_decode_workspace_bytes(w.batch, w.hq, w.hkv, w.d, w.max_seq_len, splits)
        ws = torch.full((max(nb, 16),), 0xFF, dtype=torch.uint8, device=DEV)
        out = kvq.kvq_decode_attn(cache, q, bt, sl, w.max_seq_len, w.sm_scale, workspace=ws,
                                  num_splits=splits)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert not got[0].any()
        assert_close(got, want, f"many splits d{d} hq{hq} S{splits} ({nb} workspace bytes)")


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (16, 1)])
def test_decode_group_sizes(hq, hkv):
    w = workloads.random_decode(12, batch=3, hq=hq, hkv=hkv, d=128, block=64,
                                seq_lens=[33, 200, 77])
    cache = gpu_int4_cache(w, 64)
    pool = oracle_int4_pool(w, 64)
    want = oracle.decode_int4(pool, w.hkv, w.d, 64, bits(w.q), oracle.BF16, w.block_table,
                              w.seq_lens, w.sm_scale)
    assert_close(gpu_decode(cache, w), want, f"G{hq // hkv}")


def test_decode_bf16_baseline():
    for w in (workloads.tiny_decode(1, block=0), workloads.llama8b_decode(2, batch=2, context=2048),
              workloads.random_decode(13, batch=4, hq=16, hkv=2, d=128, seq_lens=[0, 5, 40, 333])):
        cache = kvq.Bf16Cache(w.num_pages, w.hkv, w.d, DEV)
        kvq.kvq_append_paged_bf16(cache, w.k.to(DEV), w.v.to(DEV), w.slot_mapping.to(DEV))
        pool = oracle.new_bf16_pool(w.num_pages, w.hkv, w.d)
        oracle.append_bf16(pool, w.num_pages, w.hkv, w.d, bits(w.k), bits(w.v), _odt(w.k),
                           w.slot_mapping.numpy())
        want = oracle.decode_bf16(pool, w.hkv, w.d, bits(w.q), _odt(w.q), w.block_table,
                                  w.seq_lens, w.sm_scale)
        for splits in (0, 1):
            assert_close(gpu_decode(cache, w, splits, bf16=True), want, f"bf16 {w.name} S{splits}")


def test_decode_deterministic_and_page_permutation_invariant():
    w = workloads.llama8b_decode(7, batch=2, context=1000, block=64)
    cache = gpu_int4_cache(w, 64)
    a = gpu_decode(cache, w)
    b = gpu_decode(cache, w)
    assert np.array_equal(a, b)
    # move every page and its table entry together
    perm = torch.from_numpy(np.random.default_rng(3).permutation(w.num_pages)).to(DEV)
    pool2 = torch.empty_like(cache.pool)
    pool2[perm] = cache.pool
    cache2 = kvq.Int4Cache(w.num_pages, w.hkv, w.d, 64, DEV, pool=pool2)
    bt = torch.from_numpy(w.block_table).to(DEV)
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0).long()].int(), bt)
    out2 = kvq.kvq_decode_attn(cache2, w.q.to(DEV), bt2.contiguous(),
                               torch.from_numpy(w.seq_lens).to(DEV), w.max_seq_len, w.sm_scale)
    assert np.array_equal(out2.cpu().numpy().astype(np.float64), a)


def test_full_size_llama_layer_sampled():
    """The benchmark's workload at full size (64 x 4096, block 64) in the same
    launch configuration: codes of sampled sequences bit-exact, their
    attention within tolerance."""
    w = workloads.llama8b_decode(2, device=DEV, batch=64, context=4096, block=64)
    cache = kvq.Int4Cache(w.num_pages, w.hkv, w.d, 64, DEV)
    kvq.kvq_append_paged(cache, w.k, w.v, w.slot_mapping)
    out = kvq.kvq_decode_attn(cache, w.q, torch.from_numpy(w.block_table).to(DEV),
                              torch.from_numpy(w.seq_lens).to(DEV), w.max_seq_len, w.sm_scale)
    torch.cuda.synchronize()
    sample = [0, 37, 63]
    sel = torch.from_numpy(np.isin(w.token_seq, sample)).to(DEV)
    pool = oracle_int4_pool(w, 64, sel=sel)
    slab = w.hkv * oracle.int4_slab_bytes(16, w.d)
    gpool = cache.pool.cpu().numpy()
    for b in sample:
        for pg in w.block_table[b][w.block_table[b] >= 0]:
            assert np.array_equal(gpool[pg], pool[int(pg) * slab:(int(pg) + 1) * slab]), f"page {pg}"
    mask = np.zeros((w.batch, w.hq), np.uint8)
    mask[sample] = 1
    want = oracle.decode_int4(pool, w.hkv, w.d, 64, bits(w.q), oracle.BF16, w.block_table,
                              w.seq_lens, w.sm_scale, mask=mask)
    assert_close(out.cpu().numpy().astype(np.float64)[sample], want[sample], "full llama sampled")
    # two splits: 1024 workgroups, the large-grid build of the kernel
    out2 = kvq.kvq_decode_attn(cache, w.q, torch.from_numpy(w.block_table).to(DEV),
                               torch.from_numpy(w.seq_lens).to(DEV), w.max_seq_len, w.sm_scale,
                               num_splits=2)
    torch.cuda.synchronize()
    assert_close(out2.cpu().numpy().astype(np.float64)[sample], want[sample], "full llama sampled S2")


def test_decode_ignores_stale_bytes_in_unwritten_slots():
    """Pools pre-filled with 0xFF (NaN as fp16 / bf16): the slots past each
    sequence's end are never written, and must not leak into the result."""
    w = workloads.random_decode(14, batch=4, hq=8, hkv=2, d=128, block=64,
                                seq_lens=[1, 17, 30, 77])
    cache = kvq.Int4Cache(w.num_pages, w.hkv, w.d, 64, DEV)
    cache.pool.fill_(0xFF)
    kvq.kvq_append_paged(cache, w.k.to(DEV), w.v.to(DEV), w.slot_mapping.to(DEV))
    pool = oracle_int4_pool(w, 64)
    want = oracle.decode_int4(pool, w.hkv, w.d, 64, bits(w.q), oracle.BF16, w.block_table,
                              w.seq_lens, w.sm_scale)
    assert_close(gpu_decode(cache, w), want, "int4 stale")
    bc = kvq.Bf16Cache(w.num_pages, w.hkv, w.d, DEV)
    bc.pool.fill_(0xFF)
    kvq.kvq_append_paged_bf16(bc, w.k.to(DEV), w.v.to(DEV), w.slot_mapping.to(DEV))
    bpool = oracle.new_bf16_pool(w.num_pages, w.hkv, w.d)
    oracle.append_bf16(bpool, w.num_pages, w.hkv, w.d, bits(w.k), bits(w.v), oracle.BF16,
                       w.slot_mapping.numpy())
    bwant = oracle.decode_bf16(bpool, w.hkv, w.d, bits(w.q), oracle.BF16, w.block_table,
                               w.seq_lens, w.sm_scale)
    assert_close(gpu_decode(bc, w, bf16=True), bwant, "bf16 stale")


def test_append_prefill_full_size_bitexact():
    """The benchmark's prefill append at full size (32768 ragged tokens, 8 KV
    heads, head_dim 128, Student-t values, block 64): every byte of the pool."""
    w = workloads.prefill_append(3, device=DEV, block=64)
    print("append prefill full size", flush=True)
    cache = kvq.Int4Cache(w.num_pages, w.hkv, w.d, 64, DEV)
    kvq.kvq_append_paged(cache, w.k, w.v, w.slot_mapping)
    torch.cuda.synchronize()
    assert_pool_equal(cache.pool, oracle_int4_pool(w, 64), "prefill full")


def _oracle_pool_for(w, sample, step=None, kind="int4"):
    """The oracle's pool (INT4 with the workload's block, or bf16) holding
    only the tokens of the sequences in ``sample`` (of the fill ``w``, then of
    the decode ``step`` if given)."""
    def append(pool, x, sel):
        sm = x.slot_mapping.cpu().numpy()[sel]
        tsel = torch.from_numpy(sel).to(x.k.device)
        if kind == "bf16":
            oracle.append_bf16(pool, x.num_pages, x.hkv, x.d, bits(x.k[tsel]), bits(x.v[tsel]),
                               _odt(x.k), sm)
        else:
            oracle.append_int4(pool, x.num_pages, x.hkv, x.d, x.block, bits(x.k[tsel]),
                               bits(x.v[tsel]), _odt(x.k), sm)

    pool = (oracle.new_bf16_pool if kind == "bf16" else oracle.new_int4_pool)(w.num_pages, w.hkv, w.d)
    append(pool, w, np.isin(w.token_seq, sample))
    if step is not None:
        append(pool, step, np.isin(step.token_seq, sample))
    return pool


# (cache kind, Hadamard block) of the full-size sampled cases: the rotated
# and plain INT4 caches and the bf16 baseline, as the benchmark times them
FULL_KINDS = {"int4_b64": 64, "int4_plain": 0, "bf16": 0}


def _full_size_cache(kind, w, *more):
    """GPU cache of ``kind`` filled with the workload ``w`` and then the
    appends in ``more``."""
    if kind == "bf16":
        cache = kvq.Bf16Cache(w.num_pages, w.hkv, w.d, DEV)
        app = kvq.kvq_append_paged_bf16
    else:
        cache = kvq.Int4Cache(w.num_pages, w.hkv, w.d, FULL_KINDS[kind], DEV)
        app = kvq.kvq_append_paged
    for x in (w, *more):
        app(cache, x.k, x.v, x.slot_mapping)
    return cache


def _check_sampled(kind, cache, out, w, pool, sample, block_table, label):
    """Pages of the sampled sequences bit-exact (every page in their rows of
    the table: pages past a sequence's end were never written on either
    side), their attention within tolerance of the oracle's."""
    slab = w.hkv * (oracle.bf16_slab_bytes(16, w.d) if kind == "bf16" else oracle.int4_slab_bytes(16, w.d))
    for b in sample:
        pages = block_table[b][block_table[b] >= 0]
        got = cache.pool[torch.from_numpy(pages.astype(np.int64)).to(DEV)].cpu().numpy().reshape(-1)
        # (page ids as Python ints: a numpy int32 id times the slab size
        # overflows for the bf16 pools)
        want = np.concatenate([pool[int(pg) * slab:(int(pg) + 1) * slab] for pg in pages])
        assert np.array_equal(got, want), f"{label}: seq {b} pages differ"
    mask = np.zeros((w.batch, w.hq), np.uint8)
    mask[sample] = 1
    return out.cpu().numpy().astype(np.float64)[sample], mask


@pytest.mark.parametrize("kind", list(FULL_KINDS))
def test_long_context_full_size_sampled(kind):
    """Qwen3-4B-shaped long context at full size (8 x 131072 tokens, 65536
    pages, per-channel scales in [0.1, 10]) with the default split plan, for
    the rotated (block 64) and plain INT4 caches and the bf16 baseline: pages
    of two sampled sequences bit-exact, their attention within tolerance."""
    blk = FULL_KINDS[kind]
    w = workloads.long_context_decode(4, device=DEV, batch=8, context=131072, block=blk)
    print(f"long context full size {kind}", flush=True)
    cache = _full_size_cache(kind, w)
    dec = kvq.kvq_decode_attn_bf16 if kind == "bf16" else kvq.kvq_decode_attn
    out = dec(cache, w.q, torch.from_numpy(w.block_table).to(DEV), torch.from_numpy(w.seq_lens).to(DEV),
              w.max_seq_len, w.sm_scale)
    torch.cuda.synchronize()
    sample = [0, 5]
    pool = _oracle_pool_for(w, sample, kind="bf16" if kind == "bf16" else "int4")
    got, mask = _check_sampled(kind, cache, out, w, pool, sample, w.block_table, f"long {kind}")
    del cache
    if kind == "bf16":
        want = oracle.decode_bf16(pool, w.hkv, w.d, bits(w.q), oracle.BF16, w.block_table,
                                  w.seq_lens, w.sm_scale, mask=mask)
    else:
        want = oracle.decode_int4(pool, w.hkv, w.d, blk, bits(w.q), oracle.BF16, w.block_table,
                                  w.seq_lens, w.sm_scale, mask=mask)
    assert_close(got, want[sample], f"long full sampled {kind}")


@pytest.mark.parametrize("kind", list(FULL_KINDS))
def test_concurrency_full_size_sampled(kind):
    """70B-shaped layer (GQA 8) at the largest batch of the sweep: 256 ragged
    lognormal contexts (median 2048, cap 32768), one appended token per
    sequence, then decode, for the rotated (block 64) and plain INT4 caches
    and the bf16 baseline.  Sampled sequences (the longest, the shortest and
    two more): pages bit-exact, attention within tolerance."""
    blk = FULL_KINDS[kind]
    fill, steps = workloads.concurrency_step(5, device=DEV, batch=256, block=blk, steps=1)
    step = steps[0]
    print(f"concurrency full size {kind}: {int(fill.seq_lens.sum())} tokens", flush=True)
    cache = _full_size_cache(kind, fill, step)
    dec = kvq.kvq_decode_attn_bf16 if kind == "bf16" else kvq.kvq_decode_attn
    out = dec(cache, step.q, torch.from_numpy(step.block_table).to(DEV),
              torch.from_numpy(step.seq_lens).to(DEV), step.max_seq_len, step.sm_scale)
    torch.cuda.synchronize()
    lens = fill.seq_lens
    sample = sorted({int(np.argmax(lens)), int(np.argmin(lens)), 17, 200})
    pool = _oracle_pool_for(fill, sample, step=step, kind="bf16" if kind == "bf16" else "int4")
    got, mask = _check_sampled(kind, cache, out, step, pool, sample, step.block_table, f"conc {kind}")
    del cache
    if kind == "bf16":
        want = oracle.decode_bf16(pool, step.hkv, step.d, bits(step.q), oracle.BF16, step.block_table,
                                  step.seq_lens, step.sm_scale, mask=mask)
    else:
        want = oracle.decode_int4(pool, step.hkv, step.d, blk, bits(step.q), oracle.BF16,
                                  step.block_table, step.seq_lens, step.sm_scale, mask=mask)
    assert_close(got, want[sample], f"concurrency sampled {kind}")


# ---------------------------------------------------------------- high-precision windows

def _gpu_window(w, w_sink, w_recent, seed=21, final_len=None):
    """bf16 window pools (GPU and oracle) holding each sequence's window
    tokens at final_len (default: the workload's lengths)."""
    rng = np.random.default_rng(seed)
    wbt, npages = workloads.window_layout(w.batch, w_sink, w_recent, rng)
    flen = w.seq_lens if final_len is None else np.asarray(final_len)
    slots = workloads.window_slots(wbt, w.token_seq, w.token_pos, flen, w_sink, w_recent)
    win = kvq.Bf16Cache(npages, w.hkv, w.d, DEV)
    kvq.kvq_append_paged_bf16(win, w.k.to(DEV), w.v.to(DEV), torch.from_numpy(slots).to(DEV))
    pool = oracle.new_bf16_pool(npages, w.hkv, w.d)
    oracle.append_bf16(pool, npages, w.hkv, w.d, bits(w.k), bits(w.v), _odt(w.k), slots)
    return win, pool, wbt


def _windowed(cache, win, w, wbt, w_sink, w_recent, num_splits=0):
    out = kvq.kvq_decode_attn_windowed(cache, win, w.q.to(DEV), torch.from_numpy(w.block_table).to(DEV),
                                       torch.from_numpy(wbt).to(DEV), torch.from_numpy(w.seq_lens).to(DEV),
                                       w.max_seq_len, w_sink, w_recent, w.sm_scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("w_sink,w_recent", [(4, 12), (0, 20), (7, 0), (0, 0)])
def test_windowed_decode_tiny(w_sink, w_recent):
    w = workloads.tiny_decode(1, block=64)
    cache = gpu_int4_cache(w, 64)
    pool = oracle_int4_pool(w, 64)
    win, wpool, wbt = _gpu_window(w, w_sink, w_recent)
    want = oracle.decode_windowed(pool, wpool, w.hkv, w.d, 64, bits(w.q), oracle.F16, w.block_table, wbt,
                                  w.seq_lens, w_sink, w_recent, w.sm_scale)
    for splits in (0, 1, 3):
        assert_close(_windowed(cache, win, w, wbt, w_sink, w_recent, splits), want,
                     f"windowed tiny {w_sink}/{w_recent} S{splits}")


def test_windowed_decode_llama_shape():
    """Sink 4 + recent 124 tokens (128 in all, as in InnerQ Figure 5) over
    4096-token contexts, Hadamard block 64."""
    w = workloads.llama8b_decode(2, batch=3, context=4096, block=64)
    cache = gpu_int4_cache(w, 64)
    pool = oracle_int4_pool(w, 64)
    win, wpool, wbt = _gpu_window(w, 4, 124)
    want = oracle.decode_windowed(pool, wpool, w.hkv, w.d, 64, bits(w.q), oracle.BF16, w.block_table, wbt,
                                  w.seq_lens, 4, 124, w.sm_scale)
    assert_close(_windowed(cache, win, w, wbt, 4, 124), want, "windowed llama")


@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.float16)])
def test_windowed_decode_edge_lengths(d, dtype):
    lens = [0, 1, 3, 4, 5, 16, 100, 128, 129, 300]
    w = workloads.random_decode(31, batch=len(lens), hq=8, hkv=2, d=d, block=d // 2, dtype=dtype,
                                seq_lens=lens)
    cache = gpu_int4_cache(w, w.block)
    pool = oracle_int4_pool(w, w.block)
    win, wpool, wbt = _gpu_window(w, 4, 124)
    want = oracle.decode_windowed(pool, wpool, w.hkv, w.d, w.block, bits(w.q), _odt(w.q), w.block_table,
                                  wbt, w.seq_lens, 4, 124, w.sm_scale)
    for splits in (0, 1, 2, 5):
        got = _windowed(cache, win, w, wbt, 4, 124, splits)
        assert not got[0].any()                      # empty sequence -> zeros
        assert_close(got, want, f"windowed edges d{d} S{splits}")


def test_windowed_decode_ring_after_steps():
    """70B-shaped layer: fill, then decode steps that append one token per
    sequence to the INT4 cache and to the window ring, which overwrites the
    token leaving the window."""
    w_sink, w_recent = 4, 60
    fill, steps = workloads.concurrency_step(5, batch=6, block=64, steps=20, cap=2048)
    last = steps[-1]
    cache = gpu_int4_cache(fill, 64)
    rng = np.random.default_rng(22)
    wbt, npages = workloads.window_layout(fill.batch, w_sink, w_recent, rng)
    win = kvq.Bf16Cache(npages, fill.hkv, fill.d, DEV)
    wpool = oracle.new_bf16_pool(npages, fill.hkv, fill.d)
    pool = oracle_int4_pool(fill, 64)
    slots = workloads.window_slots(wbt, fill.token_seq, fill.token_pos, fill.seq_lens, w_sink, w_recent)
    kvq.kvq_append_paged_bf16(win, fill.k.to(DEV), fill.v.to(DEV), torch.from_numpy(slots).to(DEV))
    oracle.append_bf16(wpool, npages, fill.hkv, fill.d, bits(fill.k), bits(fill.v), oracle.BF16, slots)
    for st in steps:
        kvq.kvq_append_paged(cache, st.k.to(DEV), st.v.to(DEV), st.slot_mapping.to(DEV))
        oracle.append_int4(pool, st.num_pages, st.hkv, st.d, 64, bits(st.k), bits(st.v), oracle.BF16,
                           st.slot_mapping.numpy())
        s = workloads.window_slots(wbt, st.token_seq, st.token_pos, st.seq_lens, w_sink, w_recent)
        kvq.kvq_append_paged_bf16(win, st.k.to(DEV), st.v.to(DEV), torch.from_numpy(s).to(DEV))
        oracle.append_bf16(wpool, npages, st.hkv, st.d, bits(st.k), bits(st.v), oracle.BF16, s)
    want = oracle.decode_windowed(pool, wpool, last.hkv, last.d, 64, bits(last.q), oracle.BF16,
                                  last.block_table, wbt, last.seq_lens, w_sink, w_recent, last.sm_scale)
    assert_close(_windowed(cache, win, last, wbt, w_sink, w_recent), want, "windowed ring")
