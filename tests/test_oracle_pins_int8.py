"""Pins of the oracle's token-wise INT8 variant ("GPU-Accelerated INT8
Quantization for KV Cache Compression in Large Language Models", Abstract:
8-bit KV codes; the quantizer's form is the INT4 one with 255 levels) against
brute force, worked closed forms, an independent reading of the INT8 slab
layout and scipy softmax attention.  CPU only."""
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


def _vectors(rng, n=300, d=128):
    out = []
    for i in range(n):
        kind = i % 3
        if kind == 0:
            x = rng.standard_normal(d)
        elif kind == 1:
            x = rng.standard_t(3, d)
        else:
            x = rng.standard_normal(d)
            x[rng.choice(d, 4, replace=False)] *= 15
        out.append(np.float32(x))
    return out


@pytest.mark.parametrize("b", [0, 64])
def test_int8_reconstruction_error_bound(b):
    """|y - x_hat| <= s/2 inside the grid; the clamps at the ends add at most
    |min - zero| (bottom) and 255|s_exact - s| + |min - zero| (top)."""
    rng = np.random.default_rng(31)
    for x in _vectors(rng):
        y = oracle.rotate(x, b)
        codes, sh, zh = oracle.quantize(y, 8)
        s, z = _f16(sh), _f16(zh)
        y64 = y.astype(np.float64)
        err = np.abs(y64 - (codes * s + z)).max()
        mn, mx = y64.min(), y64.max()
        slop = 4 * np.spacing(np.float32(np.abs(y).max()))
        assert err <= s / 2 + abs(mn - z) + 255 * abs((mx - mn) / 255 - s) + slop
        # 8-bit codes: the error is about 1/17 of the 4-bit error on the same vector
        c4, sh4, zh4 = oracle.quantize(y, 4)
        err4 = np.abs(y64 - (c4 * _f16(sh4) + _f16(zh4))).max()
        assert err < err4 / 8


def test_int8_codes_are_nearest_grid_level():
    """Brute force over the 256 levels in fp64, away from exact half-way points."""
    rng = np.random.default_rng(32)
    checked = 0
    for x in _vectors(rng, 120):
        y = oracle.rotate(x, 32)
        codes, sh, zh = oracle.quantize(y, 8)
        s, z = _f16(sh), _f16(zh)
        levels = z + s * np.arange(256)
        for c, yy in zip(codes, y.astype(np.float64)):
            u = (yy - z) / s
            if abs(u - np.floor(u) - 0.5) < 1e-4:
                continue
            assert c == int(np.argmin(np.abs(levels - yy)))
            checked += 1
    assert checked > 12000


def test_int8_ties_round_half_to_even():
    # zero 0 and scale 1 (y spans 0..255): 2.5 -> 2, 3.5 -> 4, 254.5 -> 254, 128.5 -> 128
    y = np.zeros(64, np.float32)
    y[1] = 255.0
    y[2:6] = [2.5, 3.5, 254.5, 128.5]
    codes, sh, zh = oracle.quantize(y, 8)
    assert (sh, zh) == (0x3c00, 0x0000)
    assert codes[2:6].tolist() == [2, 4, 254, 128]


def test_int8_worked_closed_form_exact_grid():
    """y = z + k*s with z = -1 and s = 2^-7 exact in fp16, k spanning 0..255:
    the codes are k and the decoded values equal y exactly."""
    rng = np.random.default_rng(33)
    k = rng.integers(0, 256, 128)
    k[5], k[99] = 0, 255
    y = np.float32(-1.0 + k / 128.0)
    codes, sh, zh = oracle.quantize(y, 8)
    assert sh == 0x2000 and zh == 0xbc00
    assert np.array_equal(codes, k)
    assert np.array_equal(codes / 128.0 - 1.0, y.astype(np.float64))


@pytest.mark.parametrize("val", [0.0, -0.0, 3.25, -7.0])
def test_int8_constant_vector(val):
    codes, sh, zh = oracle.quantize(np.full(128, val, np.float32), 8)
    assert sh == 0 and not codes.any()
    assert zh == np.float32(val + np.float32(0.0)).astype(np.float16).view(np.uint16)


def _layout_read8(pool, hkv, d, page, head, off, kind, c, p=16):
    """Independent decoder of the INT8 slab layout (written from its text)."""
    base = (page * hkv + head) * p * (2 * d + 8)
    if kind == 0:
        code = pool[base + off * d + c]
    else:
        n, h, j = c // 8, (c % 8) // 4, c % 4
        code = pool[base + p * d + ((n * p + off) * 2 + h) * 4 + j]
    m = base + 2 * p * d + kind * 4 * p + off * 4
    return int(code), int(pool[m]) | int(pool[m + 1]) << 8, int(pool[m + 2]) | int(pool[m + 3]) << 8


@pytest.mark.parametrize("d,b", [(64, 64), (128, 16), (128, 0)])
def test_int8_append_writes_the_documented_layout(d, b):
    rng = np.random.default_rng(34)
    hkv, pages, t = 2, 4, 13
    k = rng.standard_normal((t, hkv, d)).astype(np.float16).view(np.uint16)
    v = (rng.standard_t(3, (t, hkv, d)) * 2).astype(np.float16).view(np.uint16)
    slots = rng.permutation(pages * 16)[:t].astype(np.int32)
    slots[2] = -1
    pool = oracle.new_int8_pool(pages, hkv, d, fill=0xCD)
    assert pool.size == pages * hkv * 16 * (2 * d + 8)
    oracle.append_int8(pool, pages, hkv, d, b, k, v, oracle.F16, slots)
    for ti in range(t):
        if slots[ti] < 0:
            continue
        page, off = divmod(int(slots[ti]), 16)
        for h in range(hkv):
            for kind, src in ((0, k), (1, v)):
                codes, sh, zh = oracle.quantize(oracle.rotate(src[ti, h].view(np.float16).astype(np.float32), b), 8)
                for c in range(d):
                    got = _layout_read8(pool, hkv, d, page, h, off, kind, c)
                    assert got == (codes[c], sh, zh)
                    val, c2, s2, z2 = oracle.int8_read(pool, hkv, d, page, h, off, kind, c)
                    assert (c2, s2, z2) == got and val == codes[c] * _f16(sh) + _f16(zh)
    written = set(int(s) for s in slots if s >= 0)
    page, off = divmod([s for s in range(pages * 16) if s not in written][0], 16)
    assert _layout_read8(pool, hkv, d, page, 1, off, 1, 5) == (0xCD, 0xCDCD, 0xCDCD)


def _tiny8(seed, block, lens):
    w = workloads.random_decode(seed, batch=3, hq=8, hkv=2, d=64, block=block,
                                dtype=torch.float16, seq_lens=lens)
    pool = oracle.new_int8_pool(w.num_pages, w.hkv, w.d)
    oracle.append_int8(pool, w.num_pages, w.hkv, w.d, block, workloads.bits(w.k),
                       workloads.bits(w.v), oracle.F16, w.slot_mapping.numpy())
    return w, pool


@pytest.mark.parametrize("block", [0, 32])
def test_int8_attention_matches_scipy_softmax(block):
    """Rows decoded through the layout text, rotated back with scipy's
    Hadamard, attended with scipy's softmax."""
    w, pool = _tiny8(4, block, [45, 16, 3])
    out = oracle.decode_int8(pool, w.hkv, w.d, block, workloads.bits(w.q), oracle.F16,
                             w.block_table, w.seq_lens, w.sm_scale)
    g = w.hq // w.hkv
    rinv = np.eye(w.d) if block == 0 else np.kron(np.eye(w.d // block), scipy.linalg.hadamard(block)) / np.sqrt(block)
    qf = w.q.float().numpy().astype(np.float64)

    def rows(b, kvh, kind):
        r = []
        for t in range(int(w.seq_lens[b])):
            page = int(w.block_table[b, t // 16])
            r.append([(lambda c_s_z: c_s_z[0] * _f16(c_s_z[1]) + _f16(c_s_z[2]))(
                _layout_read8(pool, w.hkv, w.d, page, kvh, t % 16, kind, c)) for c in range(w.d)])
        return np.array(r) @ rinv.T

    for b in range(w.batch):
        for h in range(w.hq):
            kk, vv = rows(b, h // g, 0), rows(b, h // g, 1)
            p = scipy.special.softmax(w.sm_scale * kk @ qf[b, h])
            assert np.abs(out[b, h] - p @ vv).max() <= 1e-12 * max(1.0, np.abs(vv).max())


def test_int8_attention_closer_to_exact_than_int4():
    """Quality proxy, not parity: against exact attention over the unquantized
    K/V, 8-bit codes err well below 4-bit codes (same rotation)."""
    w = workloads.random_decode(6, batch=2, hq=8, hkv=2, d=64, block=64, dtype=torch.float16,
                                seq_lens=[200, 120])
    p8 = oracle.new_int8_pool(w.num_pages, w.hkv, w.d)
    p4 = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
    kb, vb = workloads.bits(w.k), workloads.bits(w.v)
    sm = w.slot_mapping.numpy()
    oracle.append_int8(p8, w.num_pages, w.hkv, w.d, 64, kb, vb, oracle.F16, sm)
    oracle.append_int4(p4, w.num_pages, w.hkv, w.d, 64, kb, vb, oracle.F16, sm)
    q = workloads.bits(w.q)
    o8 = oracle.decode_int8(p8, w.hkv, w.d, 64, q, oracle.F16, w.block_table, w.seq_lens, w.sm_scale)
    o4 = oracle.decode_int4(p4, w.hkv, w.d, 64, q, oracle.F16, w.block_table, w.seq_lens, w.sm_scale)
    # exact attention over the fp16 inputs, token order = slot order of each sequence
    g = w.hq // w.hkv
    kf, vf, qf = (x.float().numpy().astype(np.float64) for x in (w.k, w.v, w.q))
    e8 = e4 = 0.0
    for b in range(w.batch):
        toks = [int(i) for i in np.flatnonzero(w.token_seq == b)]
        toks.sort(key=lambda i: int(w.token_pos[i]))
        for h in range(w.hq):
            kk, vv = kf[toks, h // g], vf[toks, h // g]
            ref = scipy.special.softmax(w.sm_scale * kk @ qf[b, h]) @ vv
            e8 = max(e8, np.abs(o8[b, h] - ref).max())
            e4 = max(e4, np.abs(o4[b, h] - ref).max())
    assert e8 < e4 / 8
