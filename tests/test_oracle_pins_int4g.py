"""Pins of the oracle's grouped INT4 variant (one fp16 scale and zero per
group of channels of the rotated vector, normally one Hadamard block; the
grouping along the inner dimension of "InnerQ", Abstract and Figure 1):
special cases that reduce to the token-wise quantizer, an independent reading
of the grouped slab layout, per-group error bounds and scipy softmax
attention.  CPU only."""
import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch

import oracle
import workloads


def setup_module(_):
    oracle.build(force=False)


def _f16(h):
    return float(np.uint16(h).view(np.float16))


def _layout_read_g(pool, hkv, d, group, page, head, off, kind, c, p=16):
    """Independent decoder of the grouped INT4 slab (written from its text)."""
    ng = d // group
    base = (page * hkv + head) * p * (d + 8 * ng)
    if kind == 0:
        byte = pool[base + off * (d // 2) + c // 2]
        code = (byte >> 4) if c % 2 else (byte & 15)
    else:
        n, j = c % (d // 8), c // (d // 8)
        byte = pool[base + p * d // 2 + (n * p + off) * 4 + j // 2]
        code = (byte >> 4) if j % 2 else (byte & 15)
    m = base + p * d + kind * 4 * p * ng + (off * ng + c // group) * 4
    return int(code), int(pool[m]) | int(pool[m + 1]) << 8, int(pool[m + 2]) | int(pool[m + 3]) << 8


def _random_tokens(rng, t, hkv, d, outliers=True):
    x = rng.standard_normal((t, hkv, d))
    if outliers:
        for h in range(hkv):
            x[:, h, rng.choice(d, 3, replace=False)] *= 20
    return x.astype(np.float16)


@pytest.mark.parametrize("d,block,group", [(128, 64, 64), (128, 32, 32), (128, 0, 32), (64, 16, 16),
                                           (64, 64, 32)])
def test_grouped_append_writes_the_documented_layout(d, block, group):
    """Every group's codes and sidecar are the token-wise quantizer applied to
    that group's slice of the rotated vector alone."""
    rng = np.random.default_rng(41)
    hkv, pages, t = 2, 4, 11
    k = _random_tokens(rng, t, hkv, d)
    v = _random_tokens(rng, t, hkv, d)
    slots = rng.permutation(pages * 16)[:t].astype(np.int32)
    slots[1] = -1
    pool = oracle.new_int4g_pool(pages, hkv, d, group, fill=0x5A)
    assert pool.size == pages * hkv * 16 * (d + 8 * (d // group))
    oracle.append_int4g(pool, pages, hkv, d, block, group, k.view(np.uint16), v.view(np.uint16),
                        oracle.F16, slots)
    for ti in range(t):
        if slots[ti] < 0:
            continue
        page, off = divmod(int(slots[ti]), 16)
        for h in range(hkv):
            for kind, src in ((0, k), (1, v)):
                y = oracle.rotate(src[ti, h].astype(np.float32), block)
                for gi in range(d // group):
                    codes, sh, zh = oracle.quantize(y[gi * group:(gi + 1) * group])
                    for c in range(group):
                        ch = gi * group + c
                        got = _layout_read_g(pool, hkv, d, group, page, h, off, kind, ch)
                        assert got == (codes[c], sh, zh)
                        val, c2, s2, z2 = oracle.int4g_read(pool, hkv, d, group, page, h, off, kind, ch)
                        assert (c2, s2, z2) == got and val == codes[c] * _f16(sh) + _f16(zh)
    written = set(int(s) for s in slots if s >= 0)
    page, off = divmod([s for s in range(pages * 16) if s not in written][0], 16)
    assert _layout_read_g(pool, hkv, d, group, page, 0, off, 1, 3)[1:] == (0x5A5A, 0x5A5A)


def test_one_group_per_vector_decodes_like_token_wise_int4():
    """group = D: the same decoded K and V as the token-wise INT4 pool."""
    rng = np.random.default_rng(42)
    d, hkv, pages, t, b = 128, 2, 3, 40, 64
    k, v = _random_tokens(rng, t, hkv, d), _random_tokens(rng, t, hkv, d)
    slots = rng.permutation(pages * 16)[:t].astype(np.int32)
    pg = oracle.new_int4g_pool(pages, hkv, d, d)
    p4 = oracle.new_int4_pool(pages, hkv, d)
    oracle.append_int4g(pg, pages, hkv, d, b, d, k.view(np.uint16), v.view(np.uint16), oracle.F16, slots)
    oracle.append_int4(p4, pages, hkv, d, b, k.view(np.uint16), v.view(np.uint16), oracle.F16, slots)
    assert pg.size == p4.size
    for s in slots[:8]:
        page, off = divmod(int(s), 16)
        for kind in (0, 1):
            for c in range(0, d, 5):
                assert oracle.int4g_read(pg, hkv, d, d, page, 1, off, kind, c) == \
                    oracle.int4_read(p4, hkv, d, page, 1, off, kind, c)


@pytest.mark.parametrize("group", [32, 64])
def test_grouped_error_bound_and_outlier_containment(group):
    """Each element is within its own group's scale/2 (plus the fp16 zero's
    rounding and fp32 slack); a group's scale never exceeds the token-wise
    scale of the whole vector (a sub-range, and fp16 rounding is monotone);
    on vectors with one outlier the RMS error drops well below the token-wise
    one, since only the outlier's group keeps a large scale."""
    rng = np.random.default_rng(43)
    d = 128
    better = 0
    for _ in range(200):
        x = rng.standard_normal(d)
        x[rng.integers(d)] *= 30
        y = oracle.rotate(np.float32(x), 0)
        y64 = y.astype(np.float64)
        sq_g = 0.0
        c4, s4, z4 = oracle.quantize(y)
        for gi in range(d // group):
            sl = slice(gi * group, (gi + 1) * group)
            codes, sh, zh = oracle.quantize(y[sl])
            s, z = _f16(sh), _f16(zh)
            err = np.abs(y64[sl] - (codes * s + z))
            mn, mx = y64[sl].min(), y64[sl].max()
            slop = 4 * np.spacing(np.float32(np.abs(y[sl]).max()))
            assert err.max() <= s / 2 + abs(mn - z) + 15 * abs((mx - mn) / 15 - s) + slop
            assert s <= _f16(s4)
            sq_g += (err ** 2).sum()
        sq_t = ((y64 - (c4 * _f16(s4) + _f16(z4))) ** 2).sum()
        better += sq_g < (group / d + 0.15) * sq_t   # about the outlier group's share of channels
    assert better > 150


@pytest.mark.parametrize("block,group", [(0, 32), (64, 64)])
def test_grouped_attention_matches_scipy_softmax(block, group):
    w = workloads.random_decode(44, batch=3, hq=8, hkv=2, d=128, block=block,
                                dtype=torch.float16, seq_lens=[40, 16, 3])
    pool = oracle.new_int4g_pool(w.num_pages, w.hkv, w.d, group)
    oracle.append_int4g(pool, w.num_pages, w.hkv, w.d, block, group, workloads.bits(w.k),
                        workloads.bits(w.v), oracle.F16, w.slot_mapping.numpy())
    out = oracle.decode_int4g(pool, w.hkv, w.d, block, group, workloads.bits(w.q), oracle.F16,
                              w.block_table, w.seq_lens, w.sm_scale)
    g = w.hq // w.hkv
    rinv = np.eye(w.d) if block == 0 else np.kron(np.eye(w.d // block), scipy.linalg.hadamard(block)) / np.sqrt(block)
    qf = w.q.float().numpy().astype(np.float64)

    def rows(b, kvh, kind):
        r = []
        for t in range(int(w.seq_lens[b])):
            page = int(w.block_table[b, t // 16])
            vals = []
            for c in range(w.d):
                code, s, z = _layout_read_g(pool, w.hkv, w.d, group, page, kvh, t % 16, kind, c)
                vals.append(code * _f16(s) + _f16(z))
            r.append(vals)
        return np.array(r) @ rinv.T

    for b in range(w.batch):
        for h in range(w.hq):
            kk, vv = rows(b, h // g, 0), rows(b, h // g, 1)
            p = scipy.special.softmax(w.sm_scale * kk @ qf[b, h])
            assert np.abs(out[b, h] - p @ vv).max() <= 1e-12 * max(1.0, np.abs(vv).max())
