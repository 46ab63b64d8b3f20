"""Pins of the oracle's MXFP4 variant (E2M1 codes with one E8M0 scale per 32
channels of the rotated vector; "BitDecoding-FP4", Abstract, for an FP4 KV
cache with Hadamard rotation under token-wise scaling): the E2M1 value table
derived from its bit fields, rounding by brute force, the shared exponent
against numpy's log2, a worked exact block, error bounds, an independent
reading of the slab layout and scipy softmax attention.  CPU only."""
import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch

import oracle
import workloads


def setup_module(_):
    oracle.build(force=False)


def _e2m1_from_bits(code):
    """E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = (m / 2.0) if e == 0 else 2.0 ** (e - 1) * (1 + m / 2.0)
    return -mag if s else mag


def test_e2m1_decode_table_from_bit_fields():
    for code in range(16):
        assert oracle.e2m1_decode(code) == _e2m1_from_bits(code)
    assert sorted({abs(_e2m1_from_bits(c)) for c in range(16)}) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e2m1_encode_is_nearest_with_ties_to_even_and_saturation():
    mags = np.array([_e2m1_from_bits(c) for c in range(8)])
    rng = np.random.default_rng(51)
    vals = list(rng.uniform(-9, 9, 4000)) + [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.99, -0.25,
                                             -5.0, -0.0, 1e-30, 0.0]
    for v in vals:
        v = float(np.float32(v))
        code = oracle.e2m1_encode(v)
        a = abs(v)
        if a >= 6:
            want = 7
        else:
            d = np.abs(mags - a)
            cands = np.flatnonzero(d == d.min())
            want = int(cands[0]) if len(cands) == 1 else int([c for c in cands if c % 2 == 0][0])
        assert code & 7 == want, (v, code)
        assert (code >> 3) == (1 if (v < 0 and want != 0) else 0), (v, code)


def test_shared_exponent_matches_log2_and_keeps_values_below_8():
    rng = np.random.default_rng(52)
    for _ in range(500):
        y = np.float32(rng.standard_normal(32) * 10.0 ** rng.uniform(-6, 4))
        codes, e = oracle.quantize_mx(y)
        x = int(np.floor(np.log2(np.abs(y).max()))) - 2
        assert e == x + 127
        v = np.abs(y.astype(np.float64)) / 2.0 ** x
        assert v.max() < 8 and v.max() >= 4
    codes, e = oracle.quantize_mx(np.zeros(32, np.float32))
    assert e == 0 and not codes.any()


def test_worked_exact_block():
    """Values that are E2M1 values times 2^5, with the block max 6 * 2^5:
    X = 5 and every element decodes exactly."""
    base = np.array([6, 4, 3, 2, 1.5, 1, 0.5, 0, -6, -4, -3, -0.5] * 2 + [6, 1, -1, 2, 3, 0.5, -2, 4])
    y = np.float32(base * 32)
    codes, e = oracle.quantize_mx(y)
    assert e == 127 + 5
    assert np.array_equal([oracle.e2m1_decode(c) * 32 for c in codes], y.astype(np.float64))


def test_mx_error_bound():
    """|y - y_hat| is at most half the E2M1 spacing around |y| / 2^X (times
    2^X), or the saturation excess above 6 * 2^X."""
    spacing = {0: 0.5, 1: 0.5, 2: 0.5, 3: 0.5, 4: 1.0, 5: 1.0, 6: 2.0, 7: 2.0}
    rng = np.random.default_rng(53)
    for _ in range(300):
        y = np.float32(rng.standard_t(3, 32))
        codes, e = oracle.quantize_mx(y)
        sc = 2.0 ** (e - 127)
        for yy, c in zip(y.astype(np.float64), codes):
            v = abs(yy) / sc
            err = abs(yy - oracle.e2m1_decode(c) * sc) / sc
            if v > 6:
                assert err <= v - 6 + 1e-12
            else:
                lo = max([m for m in (0, 0.5, 1, 1.5, 2, 3, 4, 6) if m <= v])
                assert err <= spacing[[0, 0.5, 1, 1.5, 2, 3, 4, 6].index(lo)] / 2 + 1e-12


def _layout_read_mx(pool, hkv, d, page, head, off, kind, c, p=16):
    """Independent decoder of the MXFP4 slab (written from its text)."""
    base = (page * hkv + head) * p * (d + d // 16)
    if kind == 0:
        byte = pool[base + off * (d // 2) + c // 2]
        code = (byte >> 4) if c % 2 else (byte & 15)
    else:
        n, j = c % (d // 8), c // (d // 8)
        byte = pool[base + p * d // 2 + (n * p + off) * 4 + j // 2]
        code = (byte >> 4) if j % 2 else (byte & 15)
    e = pool[base + p * d + kind * p * (d // 32) + off * (d // 32) + c // 32]
    return int(code), int(e)


@pytest.mark.parametrize("d,block", [(128, 64), (64, 0), (128, 128)])
def test_mxfp4_append_writes_the_documented_layout(d, block):
    rng = np.random.default_rng(54)
    hkv, pages, t = 2, 3, 9
    k = (rng.standard_normal((t, hkv, d)) * 3).astype(np.float16)
    v = rng.standard_t(3, (t, hkv, d)).astype(np.float16)
    slots = rng.permutation(pages * 16)[:t].astype(np.int32)
    slots[0] = -1
    pool = oracle.new_mxfp4_pool(pages, hkv, d, fill=0x77)
    assert pool.size == pages * hkv * 16 * (d + d // 16)
    oracle.append_mxfp4(pool, pages, hkv, d, block, k.view(np.uint16), v.view(np.uint16), oracle.F16, slots)
    for ti in range(1, t):
        page, off = divmod(int(slots[ti]), 16)
        for h in range(hkv):
            for kind, src in ((0, k), (1, v)):
                y = oracle.rotate(src[ti, h].astype(np.float32), block)
                for b in range(d // 32):
                    codes, e = oracle.quantize_mx(y[32 * b:32 * b + 32])
                    for c in range(32):
                        ch = 32 * b + c
                        assert _layout_read_mx(pool, hkv, d, page, h, off, kind, ch) == (codes[c], e)
                        val, c2, e2 = oracle.mxfp4_read(pool, hkv, d, page, h, off, kind, ch)
                        assert (c2, e2) == (codes[c], e) and val == oracle.e2m1_decode(codes[c]) * 2.0 ** (e - 127)


@pytest.mark.parametrize("block", [0, 64])
def test_mxfp4_attention_matches_scipy_softmax(block):
    w = workloads.random_decode(55, batch=3, hq=8, hkv=2, d=128, block=block,
                                dtype=torch.float16, seq_lens=[37, 16, 2])
    pool = oracle.new_mxfp4_pool(w.num_pages, w.hkv, w.d)
    oracle.append_mxfp4(pool, w.num_pages, w.hkv, w.d, block, workloads.bits(w.k),
                        workloads.bits(w.v), oracle.F16, w.slot_mapping.numpy())
    out = oracle.decode_mxfp4(pool, w.hkv, w.d, block, workloads.bits(w.q), oracle.F16,
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
                code, e = _layout_read_mx(pool, w.hkv, w.d, page, kvh, t % 16, kind, c)
                vals.append(_e2m1_from_bits(code) * 2.0 ** (e - 127))
            r.append(vals)
        return np.array(r) @ rinv.T

    for b in range(w.batch):
        for h in range(w.hq):
            kk, vv = rows(b, h // g, 0), rows(b, h // g, 1)
            p = scipy.special.softmax(w.sm_scale * kk @ qf[b, h])
            assert np.abs(out[b, h] - p @ vv).max() <= 1e-12 * max(1.0, np.abs(vv).max())


def test_rotation_reduces_mxfp4_key_error_on_outlier_channels():
    """Quality proxy, not parity: keys with a few outlier channels (x15) are
    reconstructed better after the Hadamard rotation (BitDecoding-FP4,
    Abstract: rotation against key outliers under token-wise scaling)."""
    rng = np.random.default_rng(56)
    d, err_plain, err_rot = 128, 0.0, 0.0
    h = np.kron(np.eye(2), scipy.linalg.hadamard(64)) / 8.0
    for _ in range(200):
        x = rng.standard_normal(d)
        x[rng.choice(d, 4, replace=False)] *= 15
        x = np.float32(x)
        for blk in (0, 64):
            y = oracle.rotate(x, blk)
            rec = np.zeros(d)
            for b in range(4):
                codes, e = oracle.quantize_mx(y[32 * b:32 * b + 32])
                rec[32 * b:32 * b + 32] = [oracle.e2m1_decode(c) * 2.0 ** (e - 127) for c in codes]
            back = rec if blk == 0 else h.T @ rec
            err = ((back - x.astype(np.float64)) ** 2).sum()
            if blk == 0:
                err_plain += err
            else:
                err_rot += err
    assert err_rot < 0.8 * err_plain
