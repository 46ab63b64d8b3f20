"""The benchmark's accuracy report reads the library's pools with its own
torch decoders of the documented page layouts (bench.dequant_pool) and
rotates the inputs with a torch block Hadamard (bench.hadamard_rotate).
Both are checked here on the CPU against pools the oracle writes and the
oracle's element reads and rotation, so the report measures what the pools
hold."""
import numpy as np
import pytest
import torch

import bench
import oracle
import workloads
from workloads import bits


def setup_module(_):
    oracle.build(force=False)


class _Pool:
    """The attributes dequant_pool reads from a cache object."""

    def __init__(self, pool, num_pages, hkv, d):
        self.pool = torch.from_numpy(pool.reshape(num_pages, -1).copy())
        self.num_pages, self.num_kv_heads, self.head_dim = num_pages, hkv, d


def _workload(d):
    return workloads.random_decode(71, batch=3, hq=8, hkv=2, d=d, block=64, seq_lens=[40, 17, 33])


def _oracle_pool(kind, w, block):
    kb, vb, sm = bits(w.k), bits(w.v), w.slot_mapping.numpy()
    if kind == "int4":
        pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
        oracle.append_int4(pool, w.num_pages, w.hkv, w.d, block, kb, vb, oracle.BF16, sm)
    elif kind == "int4_search":
        pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
        oracle.append_int4_search(pool, w.num_pages, w.hkv, w.d, block, kb, vb, oracle.BF16, sm)
    elif kind == "int8":
        pool = oracle.new_int8_pool(w.num_pages, w.hkv, w.d)
        oracle.append_int8(pool, w.num_pages, w.hkv, w.d, block, kb, vb, oracle.BF16, sm)
    elif kind == "int4g":
        pool = oracle.new_int4g_pool(w.num_pages, w.hkv, w.d, 64)
        oracle.append_int4g(pool, w.num_pages, w.hkv, w.d, block, 64, kb, vb, oracle.BF16, sm)
    elif kind == "int4g_hybrid":
        pool = oracle.new_int4g_pool(w.num_pages, w.hkv, w.d, 64)
        oracle.append_int4g_hybrid(pool, w.num_pages, w.hkv, w.d, block, 64, kb, vb, oracle.BF16, sm)
    else:
        pool = oracle.new_mxfp4_pool(w.num_pages, w.hkv, w.d)
        oracle.append_mxfp4(pool, w.num_pages, w.hkv, w.d, block, kb, vb, oracle.BF16, sm)
    return pool


def _read(kind, pool, w, page, head, off, which, c):
    if kind in ("int4", "int4_search"):
        return oracle.int4_read(pool, w.hkv, w.d, page, head, off, which, c)[0]
    if kind == "int8":
        return oracle.int8_read(pool, w.hkv, w.d, page, head, off, which, c)[0]
    if kind in ("int4g", "int4g_hybrid"):
        return oracle.int4g_read(pool, w.hkv, w.d, 64, page, head, off, which, c)[0]
    return oracle.mxfp4_read(pool, w.hkv, w.d, page, head, off, which, c)[0]


@pytest.mark.parametrize("kind", ["int4", "int4_search", "int8", "int4g", "int4g_hybrid", "mxfp4"])
@pytest.mark.parametrize("d", [128, 64])
def test_dequant_pool_matches_the_oracle_reads(kind, d):
    if kind == "mxfp4" and d == 64:
        pytest.skip("the MXFP4 pool is built for head_dim 128")
    w = _workload(d)
    pool = _oracle_pool(kind, w, 64)
    bench_kind = {"int4_search": "int4", "int4g_hybrid": "int4g"}.get(kind, kind)
    rng = np.random.default_rng(3)
    toks = rng.choice(w.num_tokens, 12, replace=False)
    slots = w.slot_mapping.numpy()[toks].astype(np.int64)
    dk, dv = bench.dequant_pool(torch, bench_kind, _Pool(pool, w.num_pages, w.hkv, d), torch.from_numpy(slots))
    for i, s in enumerate(slots):
        page, off = int(s) // 16, int(s) % 16
        for h in range(w.hkv):
            for which, got in ((0, dk), (1, dv)):
                want = np.array([_read(kind, pool, w, page, h, off, which, c) for c in range(d)])
                np.testing.assert_allclose(got[i, h].numpy(), want, rtol=1e-6, atol=1e-6 * np.abs(want).max(),
                                           err_msg=f"{kind} d{d} slot {s} head {h} {'KV'[which]}")


@pytest.mark.parametrize("block", [0, 16, 32, 64, 128])
def test_hadamard_rotate_matches_the_oracle_rotation(block):
    x = np.random.default_rng(block).standard_normal((5, 128)).astype(np.float32)
    got = bench.hadamard_rotate(torch, torch.from_numpy(x), block).numpy()
    want = np.stack([oracle.rotate(row, block) for row in x])   # the oracle rotates one vector a call
    np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-5)
