"""Pins of the CPU oracle against things other than itself: closed forms,
library routines (numpy fp16 casts, scipy's Sylvester Hadamard, scipy softmax),
exact arithmetic (decimal), brute force and invariants.  CPU only."""
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch

import oracle
import workloads

BLOCKS = [16, 32, 64, 128]


def setup_module(_):
    oracle.build(force=False)


# ---------------------------------------------------------------- formats

def _fp16_sweep():
    """fp32 inputs around every finite fp16 value: the value, the midpoints to
    its neighbours (ties) and the fp32 values just beside each midpoint."""
    h = np.arange(0, 0x7c00, dtype=np.uint16)
    v = h.view(np.float16).astype(np.float32)
    nxt = (h + 1).view(np.float16).astype(np.float32)       # 0x7c00 -> inf at the end
    mid = ((v.astype(np.float64) + np.where(np.isinf(nxt), 65536.0, nxt)) / 2).astype(np.float32)
    below = np.nextafter(mid, np.float32(0))
    above = np.nextafter(mid, np.float32(np.inf))
    xs = np.concatenate([v, mid, below, above, [65519.0, 65520.0, 65536.0, 1e9, 1e-30]]).astype(np.float32)
    return np.concatenate([xs, -xs])


def test_f32_to_f16_matches_numpy_cast():
    xs = _fp16_sweep()
    got = np.array([oracle.f32_to_f16(float(x)) for x in xs], np.uint16)
    want = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_f16_to_f32_exact_all_patterns():
    h = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (h & 0x7c00) != 0x7c00
    got = np.array([oracle.f16_to_f32(int(x)) for x in h[finite]], np.float32)
    want = h[finite].view(np.float16).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_f32_to_bf16_matches_torch_cast():
    rng = np.random.default_rng(0)
    xs = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 50,
        # exact ties between bf16 neighbours and the values beside them
        (np.arange(1, 4000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        (np.arange(1, 4000, dtype=np.uint32) << 16 | 0x7fff).view(np.float32),
        (np.arange(1, 4000, dtype=np.uint32) << 16 | 0x8001).view(np.float32),
    ]).astype(np.float32)
    xs = xs[np.isfinite(xs)]
    got = np.array([oracle.f32_to_bf16(float(x)) for x in xs], np.uint16)
    want = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("b", BLOCKS)
def test_block_scale_is_correctly_rounded_inverse_sqrt(b):
    getcontext().prec = 60
    exact = Decimal(1) / Decimal(b).sqrt()
    s = oracle.block_scale(b)
    lo, hi = np.nextafter(s, np.float32(0)), np.nextafter(s, np.float32(1))
    err = abs(Decimal(float(s)) - exact)
    assert err <= abs(Decimal(float(lo)) - exact) and err <= abs(Decimal(float(hi)) - exact)


# ---------------------------------------------------------------- rotation

def _rotation_matrix(d, b):
    """Columns = oracle rotation of the unit vectors."""
    eye = np.eye(d, dtype=np.float32)
    return np.stack([oracle.rotate(eye[j], b) for j in range(d)], axis=1)


@pytest.mark.parametrize("b", BLOCKS)
def test_rotation_of_unit_vectors_is_sylvester_hadamard(b):
    d = 128
    r = _rotation_matrix(d, b)
    h = scipy.linalg.hadamard(b).astype(np.float32)
    want = np.kron(np.eye(d // b, dtype=np.float32), h) * oracle.block_scale(b)
    assert np.array_equal(r, want)          # FWHT of e_j is exact; x s_b is one rounding


@pytest.mark.parametrize("b", BLOCKS)
def test_rotation_is_orthonormal(b):
    r = _rotation_matrix(128, b).astype(np.float64)
    assert np.abs(r @ r.T - np.eye(128)).max() <= 4e-8


@pytest.mark.parametrize("b", BLOCKS)
def test_rotation_matches_fp64_matrix_product(b):
    rng = np.random.default_rng(b)
    d = 128
    h = np.kron(np.eye(d // b), scipy.linalg.hadamard(b)) / np.sqrt(b)
    for _ in range(50):
        x = (rng.standard_normal(d) * rng.choice([0.1, 1, 30], d)).astype(np.float32)
        y = oracle.rotate(x, b).astype(np.float64)
        y64 = h @ x.astype(np.float64)
        # fp32 butterfly: log2(b) roundings of partial sums bounded by |x|_1
        bound = (np.log2(b) + 2) * 2.0 ** -24 * np.abs(x).sum()
        assert np.abs(y - y64).max() <= bound


@pytest.mark.parametrize("b", BLOCKS)
def test_rotated_dot_product_preserved(b):
    rng = np.random.default_rng(100 + b)
    for _ in range(200):
        q = rng.standard_normal(128).astype(np.float32)
        k = (rng.standard_normal(128) * rng.choice([1, 20], 128)).astype(np.float32)
        qr, kr = oracle.rotate(q, b).astype(np.float64), oracle.rotate(k, b).astype(np.float64)
        ref = q.astype(np.float64) @ k.astype(np.float64)
        assert abs(qr @ kr - ref) <= 1e-5 * np.linalg.norm(q) * np.linalg.norm(k)
        assert abs(np.linalg.norm(qr) - np.linalg.norm(q)) <= 1e-6 * np.linalg.norm(q)


def test_butterfly_stage_order_worked_example():
    """The fp32 butterfly runs its stages in ascending order: a 16-element
    vector whose result differs between the two stage orders, with the
    expected bits derived by hand in the fixture (tests/golden/
    fwht_stage_order.txt)."""
    import os
    rows = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "fwht_stage_order.txt")):
        if line.startswith("#") or not line.strip():
            continue
        key, *vals = line.split()
        rows[key] = vals
    b = int(rows["block"][0])
    x = np.array([int(h, 16) for h in rows["input"]], np.uint32).view(np.float32)
    want = np.array([int(h, 16) for h in rows["output"]], np.uint32)
    got = oracle.rotate(x, b).view(np.uint32)
    assert np.array_equal(got, want), [hex(v) for v in got]


def test_block_one_is_identity_of_plain_int4():
    rng = np.random.default_rng(7)
    for _ in range(100):
        x = (rng.standard_normal(128) * 3).astype(np.float32)
        assert np.array_equal(oracle.rotate(x, 1), x)
        assert oracle.quantize(oracle.rotate(x, 1))[0].tolist() == oracle.quantize(x)[0].tolist()


# ---------------------------------------------------------------- quantizer

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
def test_reconstruction_error_bound(b):
    """|y - x_hat| <= s/2 inside the grid; the clamps at the ends add at most
    |min - zero| (bottom) and 15|s_exact - s| + |min - zero| (top)."""
    rng = np.random.default_rng(11)
    for x in _vectors(rng):
        y = oracle.rotate(x, b)
        codes, sh, zh = oracle.quantize(y)
        s, z = _f16(sh), _f16(zh)
        y64 = y.astype(np.float64)
        xhat = codes * s + z
        mn, mx = y64.min(), y64.max()
        slop = 4 * np.spacing(np.float32(np.abs(y).max()))
        bound = s / 2 + abs(mn - z) + 15 * abs((mx - mn) / 15 - s) + slop
        assert np.abs(y64 - xhat).max() <= bound
        # typical data: the fp16 rounding of the zero stays far below s/2
        assert np.abs(y64 - xhat).max() <= s / 2 + 2e-3 * s + slop


def test_codes_are_nearest_grid_level():
    """Brute force over the 16 levels with exact (fp64) arithmetic, wherever the
    exact ratio is not within 1e-5 of a half integer."""
    rng = np.random.default_rng(12)
    checked = 0
    for x in _vectors(rng, 200):
        y = oracle.rotate(x, 64)
        codes, sh, zh = oracle.quantize(y)
        s, z = _f16(sh), _f16(zh)
        levels = z + s * np.arange(16)
        for c, yy in zip(codes, y.astype(np.float64)):
            u = (yy - z) / s
            if abs(u - np.floor(u) - 0.5) < 1e-5:
                continue
            best = int(np.argmin(np.abs(levels - yy)))
            assert c == best
            checked += 1
    assert checked > 20000


def test_ties_round_half_to_even():
    # levels z=0, s=1 (y spans 0..15): y = 2.5 -> 2, 3.5 -> 4, 0.5 -> 0, 14.5 -> 14
    y = np.zeros(64, np.float32)
    y[1] = 15.0
    y[2:6] = [2.5, 3.5, 0.5, 14.5]
    codes, sh, zh = oracle.quantize(y)
    assert (sh, zh) == (0x3c00, 0x0000)
    assert codes[2:6].tolist() == [2, 4, 0, 14]


def test_worked_closed_form_exact_grid():
    """y = z + k*s with z = -1 and s = 1/8 exact in fp16 and k spanning 0..15:
    plain INT4 reproduces k and y exactly."""
    rng = np.random.default_rng(13)
    k = rng.integers(0, 16, 128)
    k[3], k[77] = 0, 15
    y = np.float32(-1.0 + k * 0.125)
    codes, sh, zh = oracle.quantize(y)
    assert sh == 0x3000 and zh == 0xbc00
    assert np.array_equal(codes, k)
    assert np.array_equal(codes * 0.125 - 1.0, y.astype(np.float64))


@pytest.mark.parametrize("val", [0.0, -0.0, 3.25, -7.0, 1e-6])
def test_constant_vector(val):
    y = np.full(128, val, np.float32)
    codes, sh, zh = oracle.quantize(y)
    assert sh == 0 and not codes.any()
    assert zh == np.float32(val + np.float32(0.0)).astype(np.float16).view(np.uint16)
    if val == 0.0:
        assert zh == 0x0000     # -0 is canonicalised to +0


def test_subnormal_scale():
    y = np.zeros(64, np.float32)
    y[5] = 1e-6                 # step 6.7e-8 -> fp16 subnormal 0x0001
    codes, sh, zh = oracle.quantize(y)
    assert sh == 0x0001 and zh == 0
    assert codes[5] == 15 and codes.sum() == 15


# ---------------------------------------------------------------- layout

def _layout_read(pool, hkv, d, page, head, off, kind, c, p=16):
    """Independent decoder of the INT4 slab layout (written from its text)."""
    slab = p * (d + 8)
    base = (page * hkv + head) * slab
    if kind == 0:
        byte = pool[base + off * (d // 2) + c // 2]
    else:
        byte = pool[base + p * d // 2 + ((c // 8) * p + off) * 4 + (c % 8) // 2]
    code = (byte >> 4) if c % 2 else (byte & 15)
    m = base + p * d + kind * 4 * p + off * 4
    scale = int(pool[m]) | int(pool[m + 1]) << 8
    zero = int(pool[m + 2]) | int(pool[m + 3]) << 8
    return int(code), scale, zero


@pytest.mark.parametrize("d,b", [(64, 64), (128, 32), (128, 0)])
def test_append_writes_the_documented_layout(d, b):
    rng = np.random.default_rng(21)
    hkv, pages, t = 3, 5, 17
    k = rng.standard_normal((t, hkv, d)).astype(np.float16).view(np.uint16)
    v = (rng.standard_normal((t, hkv, d)) * 4).astype(np.float16).view(np.uint16)
    slots = rng.permutation(pages * 16)[:t].astype(np.int32)
    slots[4] = -1                             # skipped
    pool = oracle.new_int4_pool(pages, hkv, d, fill=0xAB)
    oracle.append_int4(pool, pages, hkv, d, b, k, v, oracle.F16, slots)
    for ti in range(t):
        for h in range(hkv):
            for kind, src in ((0, k), (1, v)):
                x = src[ti, h].view(np.float16).astype(np.float32)
                codes, sh, zh = oracle.quantize(oracle.rotate(x, b))
                if slots[ti] < 0:
                    continue
                page, off = divmod(int(slots[ti]), 16)
                for c in range(d):
                    code, s, z = _layout_read(pool, hkv, d, page, h, off, kind, c)
                    assert (code, s, z) == (codes[c], sh, zh)
                    val, code2, s2, z2 = oracle.int4_read(pool, hkv, d, page, h, off, kind, c)
                    assert (code2, s2, z2) == (code, s, z)
                    assert val == code * _f16(s) + _f16(z)
    # the skipped token's slot keeps the fill pattern everywhere
    written = set(int(s) for s in slots if s >= 0)
    free = [s for s in range(pages * 16) if s not in written][0]
    page, off = divmod(free, 16)
    assert _layout_read(pool, hkv, d, page, 0, off, 0, 0)[1] == 0xABAB


def test_bf16_append_layout_and_rounding():
    rng = np.random.default_rng(22)
    hkv, d, pages, t = 2, 64, 3, 20
    x16 = rng.standard_normal((t, hkv, d)).astype(np.float16)
    slots = rng.permutation(pages * 16)[:t].astype(np.int32)
    pool = oracle.new_bf16_pool(pages, hkv, d)
    oracle.append_bf16(pool, pages, hkv, d, x16.view(np.uint16), (x16 * 2).view(np.uint16),
                       oracle.F16, slots)
    want_k = torch.from_numpy(x16.astype(np.float32)).to(torch.bfloat16).float().numpy()
    want_v = torch.from_numpy((x16 * 2).astype(np.float32)).to(torch.bfloat16).float().numpy()
    words = pool.view(np.uint16)
    for ti in range(t):
        page, off = divmod(int(slots[ti]), 16)
        for h in range(hkv):
            base = (page * hkv + h) * 2 * 16 * d
            for c in range(d):
                kb = words[base + off * d + c]
                n, j, g, i = c // 8, c % 8, off // 4, off % 4
                vb = words[base + 16 * d + ((n * 4 + g) * 8 + j) * 4 + i]
                assert np.uint32(kb).astype(np.uint32) << 16 == np.float32(want_k[ti, h, c]).view(np.uint32)
                assert np.uint32(vb) << 16 == np.float32(want_v[ti, h, c]).view(np.uint32)
                assert oracle.bf16_read(pool, hkv, d, page, h, off, 1, c) == want_v[ti, h, c]


# ---------------------------------------------------------------- attention

def _tiny_case(seed=1, block=64, lens=None):
    w = workloads.random_decode(seed, batch=3, hq=8, hkv=2, d=64, block=block,
                                dtype=torch.float16, seq_lens=lens)
    pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
    oracle.append_int4(pool, w.num_pages, w.hkv, w.d, w.block, workloads.bits(w.k),
                       workloads.bits(w.v), oracle.F16, w.slot_mapping.numpy())
    return w, pool


def _dequant_seq(w, pool, b, kvh, kind):
    rows = []
    for t in range(int(w.seq_lens[b])):
        page = int(w.block_table[b, t // 16])
        rows.append([oracle.int4_read(pool, w.hkv, w.d, page, kvh, t % 16, kind, c)[0]
                     for c in range(w.d)])
    return np.array(rows)


@pytest.mark.parametrize("block", [0, 16, 64])
def test_paged_attention_equals_bruteforce_twin(block):
    w, pool = _tiny_case(block=block, lens=[37, 16, 1])
    q = workloads.bits(w.q)
    a = oracle.decode_int4(pool, w.hkv, w.d, block, q, oracle.F16, w.block_table, w.seq_lens, w.sm_scale)
    bf = oracle.decode_int4_bruteforce(pool, w.hkv, w.d, block, q, oracle.F16, w.block_table,
                                       w.seq_lens, w.sm_scale)
    assert np.abs(a - bf).max() <= 1e-12 * max(1.0, np.abs(a).max())


@pytest.mark.parametrize("block", [0, 32])
def test_paged_attention_matches_scipy_softmax(block):
    """Decoded rows read through the documented layout, rotated back with
    scipy's Hadamard, attended with scipy's softmax."""
    w, pool = _tiny_case(seed=2, block=block, lens=[50, 23, 64])
    q = workloads.bits(w.q)
    out = oracle.decode_int4(pool, w.hkv, w.d, block, q, oracle.F16, w.block_table, w.seq_lens, w.sm_scale)
    g = w.hq // w.hkv
    rinv = np.eye(w.d) if block == 0 else np.kron(np.eye(w.d // block), scipy.linalg.hadamard(block)) / np.sqrt(block)
    qf = w.q.float().numpy().astype(np.float64)
    for b in range(w.batch):
        for h in range(w.hq):
            kk = _dequant_seq(w, pool, b, h // g, 0) @ rinv.T
            vv = _dequant_seq(w, pool, b, h // g, 1) @ rinv.T
            p = scipy.special.softmax(w.sm_scale * kk @ qf[b, h])
            assert np.abs(out[b, h] - p @ vv).max() <= 1e-12 * max(1.0, np.abs(vv).max())


def test_single_token_and_identical_keys():
    w, pool = _tiny_case(seed=3, block=64, lens=[1, 40, 5])
    q = workloads.bits(w.q)
    out = oracle.decode_int4(pool, w.hkv, w.d, 64, q, oracle.F16, w.block_table, w.seq_lens, w.sm_scale)
    rinv = np.kron(np.eye(w.d // 64), scipy.linalg.hadamard(64)) / 8.0
    g = w.hq // w.hkv
    for h in range(w.hq):        # L = 1: the output is the one decoded value, un-rotated
        v0 = _dequant_seq(w, pool, 0, h // g, 1)[0] @ rinv.T
        assert np.abs(out[0, h] - v0).max() <= 1e-12 * np.abs(v0).max()
    # identical keys everywhere -> uniform weights -> mean of the decoded values
    k = w.k.clone()
    k[:] = k[0:1, :, :]
    pool2 = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
    oracle.append_int4(pool2, w.num_pages, w.hkv, w.d, 64, workloads.bits(k), workloads.bits(w.v),
                       oracle.F16, w.slot_mapping.numpy())
    out2 = oracle.decode_int4(pool2, w.hkv, w.d, 64, q, oracle.F16, w.block_table, w.seq_lens, w.sm_scale)
    for b in range(w.batch):
        for h in range(w.hq):
            mean = (_dequant_seq(w, pool2, b, h // g, 1) @ rinv.T).mean(axis=0)
            assert np.abs(out2[b, h] - mean).max() <= 1e-12 * max(1.0, np.abs(mean).max())


def test_empty_sequence_gives_zeros():
    w, pool = _tiny_case(seed=4, block=64, lens=[0, 17, 3])
    out = oracle.decode_int4(pool, w.hkv, w.d, 64, workloads.bits(w.q), oracle.F16, w.block_table,
                             w.seq_lens, w.sm_scale)
    assert not out[0].any() and np.abs(out[1]).max() > 0


def test_absent_pages_leave_their_tokens_out():
    """A block-table entry outside [0, num_pages) (negative or past the pool)
    is a page that is not there: the row equals attention over the other
    tokens (rebuilt as a shorter sequence over the remaining pages), and a row
    whose pages are all absent is zero."""
    w, pool = _tiny_case(seed=6, block=64, lens=[40, 40, 33])
    q = workloads.bits(w.q)
    args = (w.hkv, w.d, 64, q, oracle.F16)
    bt = w.block_table.copy()
    p0, p1, p2 = (int(x) for x in bt[0][:3])
    bt[0][1] = -1                                  # the middle page of sequence 0 (tokens 16..31)
    bt[1][2] = w.num_pages + 3                     # the last page of sequence 1 (tokens 32..39)
    bt[2][:3] = [-1, -5, w.num_pages]              # every page of sequence 2
    out = oracle.decode_int4(pool, *args, bt, w.seq_lens, w.sm_scale)
    ref_bt = w.block_table.copy()
    ref_bt[0][:2] = [p0, p2]                       # tokens 0..15 then 32..39: 24 tokens
    ref_lens = np.array([24, 32, 0], np.int32)
    ref = oracle.decode_int4(pool, *args, ref_bt, ref_lens, w.sm_scale)
    assert np.allclose(out[0], ref[0], rtol=1e-12, atol=1e-14)
    assert np.array_equal(out[1], ref[1])          # the same tokens in the same order
    assert not out[2].any()
    assert np.abs(out[0] - oracle.decode_int4(pool, *args, w.block_table, w.seq_lens, w.sm_scale)[0]).max() > 1e-6


def test_page_permutation_invariance():
    """Moving pages and their table entries together leaves the output bit-identical."""
    w, pool = _tiny_case(seed=5, block=64, lens=[70, 33, 16])
    q = workloads.bits(w.q)
    out = oracle.decode_int4(pool, w.hkv, w.d, 64, q, oracle.F16, w.block_table, w.seq_lens, w.sm_scale)
    rng = np.random.default_rng(5)
    perm = rng.permutation(w.num_pages)          # new page id of old page i = perm[i]
    slab = w.hkv * oracle.int4_slab_bytes(16, w.d)
    pool2 = np.empty_like(pool)
    for old in range(w.num_pages):
        pool2[perm[old] * slab:(perm[old] + 1) * slab] = pool[old * slab:(old + 1) * slab]
    bt2 = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    out2 = oracle.decode_int4(pool2, w.hkv, w.d, 64, q, oracle.F16, bt2, w.seq_lens, w.sm_scale)
    assert np.array_equal(out, out2)


def test_split_logsumexp_combine_equals_single_pass():
    """The split-K merge (max, rescaled sums, rescaled partial outputs) that the
    GPU reduce uses is exact attention: here against scipy on decoded rows."""
    w, pool = _tiny_case(seed=6, block=0, lens=[150, 9, 64])
    q = w.q.float().numpy().astype(np.float64)
    g = w.hq // w.hkv
    for b in range(w.batch):
        kk = _dequant_seq(w, pool, b, 0, 0)
        vv = _dequant_seq(w, pool, b, 0, 1)
        s = w.sm_scale * kk @ q[b, 0]
        parts = []
        for lo in range(0, len(s), 32):
            m = s[lo:lo + 32].max()
            p = np.exp(s[lo:lo + 32] - m)
            parts.append((m, p.sum(), p @ vv[lo:lo + 32]))
        mstar = max(m for m, _, _ in parts)
        l = sum(l * np.exp(m - mstar) for m, l, _ in parts)
        o = sum(a * np.exp(m - mstar) for m, _, a in parts) / l
        ref = scipy.special.softmax(s) @ vv
        assert np.abs(o - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
        assert g == 4


def test_bf16_attention_matches_scipy():
    w = workloads.random_decode(7, batch=2, hq=4, hkv=2, d=64, block=0, dtype=torch.bfloat16,
                                seq_lens=[33, 100])
    pool = oracle.new_bf16_pool(w.num_pages, w.hkv, w.d)
    oracle.append_bf16(pool, w.num_pages, w.hkv, w.d, workloads.bits(w.k), workloads.bits(w.v),
                       oracle.BF16, w.slot_mapping.numpy())
    out = oracle.decode_bf16(pool, w.hkv, w.d, workloads.bits(w.q), oracle.BF16, w.block_table,
                             w.seq_lens, w.sm_scale)
    kf, vf, qf = (x.float().numpy().astype(np.float64) for x in (w.k, w.v, w.q))
    for b in range(w.batch):
        sel = w.token_seq == b
        for h in range(w.hq):
            p = scipy.special.softmax(w.sm_scale * kf[sel, h // 2] @ qf[b, h])
            assert np.abs(out[b, h] - p @ vf[sel, h // 2]).max() <= 1e-12


def test_rotation_reduces_error_on_outlier_data():
    """Quality proxy for the claim that the rotation recovers the accuracy lost
    by naive INT4 (outlier channels x20): attention error vs exact attention on
    the unquantized inputs is lower with the rotation."""
    w = workloads.tiny_decode(1, block=64)
    k, v, q = workloads.bits(w.k), workloads.bits(w.v), workloads.bits(w.q)
    sm = w.slot_mapping.numpy()
    errs = {}
    for b in (0, 64):
        pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
        oracle.append_int4(pool, w.num_pages, w.hkv, w.d, b, k, v, oracle.F16, sm)
        out = oracle.decode_int4(pool, w.hkv, w.d, b, q, oracle.F16, w.block_table, w.seq_lens, w.sm_scale)
        errs[b] = out
    kf, vf, qf = (x.float().numpy().astype(np.float64) for x in (w.k, w.v, w.q))
    ref = np.zeros_like(errs[0])
    for b in range(w.batch):
        sel = w.token_seq == b
        for h in range(w.hq):
            p = scipy.special.softmax(w.sm_scale * kf[sel, h // 4] @ qf[b, h])
            ref[b, h] = p @ vf[sel, h // 4]
    e_plain = np.linalg.norm(errs[0] - ref)
    e_rot = np.linalg.norm(errs[64] - ref)
    assert e_rot < 0.8 * e_plain


# ---------------------------------------------------------------- accounting

def _table3():
    rows = {}
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "innerq_table3_bitwidth.txt")
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        m, cache, qty, val = line.split()
        rows[(m, cache, qty)] = float(val)
    return rows


def test_pool_bit_widths_match_innerq_table3_accounting():
    """The oracle's page slabs hold, per stored number, the integer bits plus
    the FP16 scale and zero bits averaged over the numbers of their group --
    the accounting of InnerQ Table 3 (group 32: 0.5 bit each for scale and
    zero point, KIVI's key row).  Token-wise INT4 over head_dim 128 is then 4 +
    0.25 bits, grouped INT4 with groups of 32 is 4 + 0.5 + 0.5, and INT8 is 8 +
    0.25."""
    t3 = _table3()
    numbers = 16 * 2 * 128          # tokens of a page x (K, V) x channels
    bits_of = lambda slab: slab * 8 / numbers
    fp16_over = lambda group: 16 / group
    assert fp16_over(32) == t3[("KIVI", "key", "scale")] == t3[("KIVI", "key", "zero_point")]
    assert bits_of(oracle.int4g_slab_bytes(16, 128, 32)) == 4 + t3[("KIVI", "key", "scale")] + t3[("KIVI", "key", "zero_point")]
    assert bits_of(oracle.int4_slab_bytes(16, 128)) == 4 + 2 * fp16_over(128)
    assert bits_of(oracle.int4g_slab_bytes(16, 128, 64)) == 4 + 2 * fp16_over(64)
    assert bits_of(oracle.int8_slab_bytes(16, 128)) == 8 + 2 * fp16_over(128)
    # the same averaging gives the table's FP32 channel norm over head dim 128
    assert 32 / 128 == t3[("TurboQuant", "key", "channel_norm")]


def test_prefill_lengths_ragged_and_exact():
    rng = np.random.default_rng(np.random.SeedSequence(3003))
    lens = workloads.prefill_lengths(32768, 16, 512, 4096, rng)
    assert lens.sum() == 32768 and lens.min() >= 512 and lens.max() <= 4096
    assert len(set(lens.tolist())) > 8


def test_large_logits_stay_finite():
    """Logits far beyond exp's fp64 range (q scaled x300): the max-subtracted
    softmax must still match scipy."""
    w, pool = _tiny_case(seed=8, block=64, lens=[40, 7, 19])
    qbig = (w.q.float() * 300).to(torch.float16)
    out = oracle.decode_int4(pool, w.hkv, w.d, 64, workloads.bits(qbig), oracle.F16, w.block_table,
                             w.seq_lens, w.sm_scale)
    assert np.isfinite(out).all()
    rinv = np.kron(np.eye(w.d // 64), scipy.linalg.hadamard(64)) / 8.0
    qf = qbig.float().numpy().astype(np.float64)
    for b in range(w.batch):
        kk = _dequant_seq(w, pool, b, 0, 0) @ rinv.T
        vv = _dequant_seq(w, pool, b, 0, 1) @ rinv.T
        p = scipy.special.softmax(w.sm_scale * kk @ qf[b, 0])
        assert np.abs(out[b, 0] - p @ vv).max() <= 1e-9 * np.abs(vv).max()


# ---------------------------------------------------------------- high-precision windows

def _window_pool(w, w_sink, w_recent, seed=5, final_len=None):
    """The bf16 window pool holding, for each sequence, the tokens that are in
    its windows at length final_len (default: the workload's lengths)."""
    rng = np.random.default_rng(seed)
    wbt, npages = workloads.window_layout(w.batch, w_sink, w_recent, rng)
    flen = w.seq_lens if final_len is None else np.asarray(final_len)
    slots = workloads.window_slots(wbt, w.token_seq, w.token_pos, flen, w_sink, w_recent)
    pool = oracle.new_bf16_pool(npages, w.hkv, w.d)
    oracle.append_bf16(pool, npages, w.hkv, w.d, workloads.bits(w.k), workloads.bits(w.v),
                       oracle.F16 if w.k.dtype == torch.float16 else oracle.BF16, slots)
    return wbt, pool


def test_windowed_without_windows_is_int4_attention():
    w, pool = _tiny_case(seed=6, block=64, lens=[45, 16, 3])
    wbt, wpool = _window_pool(w, 0, 0)
    q = workloads.bits(w.q)
    a = oracle.decode_int4(pool, w.hkv, w.d, 64, q, oracle.F16, w.block_table, w.seq_lens, w.sm_scale)
    b = oracle.decode_windowed(pool, wpool, w.hkv, w.d, 64, q, oracle.F16, w.block_table, wbt,
                               w.seq_lens, 0, 0, w.sm_scale)
    assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(a).max())


@pytest.mark.parametrize("w_sink,w_recent", [(64, 0), (0, 64), (20, 44)])
def test_windowed_covering_everything_is_bf16_attention(w_sink, w_recent):
    """Windows at least as long as every sequence: every token is read as
    bf16, which is plain bf16 attention over the window pool."""
    w, pool = _tiny_case(seed=7, block=32, lens=[40, 64, 9])
    wbt, wpool = _window_pool(w, w_sink, w_recent)
    q = workloads.bits(w.q)
    want = oracle.decode_bf16(wpool, w.hkv, w.d, q, oracle.F16, wbt, w.seq_lens, w.sm_scale)
    got = oracle.decode_windowed(pool, wpool, w.hkv, w.d, 32, q, oracle.F16, w.block_table, wbt,
                                 w.seq_lens, w_sink, w_recent, w.sm_scale)
    assert np.abs(got - want).max() <= 1e-12 * max(1.0, np.abs(want).max())


@pytest.mark.parametrize("block,w_sink,w_recent", [(64, 4, 12), (16, 0, 20), (0, 7, 0)])
def test_windowed_matches_explicit_rows(block, w_sink, w_recent):
    """Brute force: each token's key and value assembled by hand (window
    tokens from the inputs rounded to bf16 by torch, the others decoded from
    the INT4 pool and rotated back with scipy's Hadamard), one scipy softmax."""
    w, pool = _tiny_case(seed=8, block=block, lens=[53, 21, 6])
    wbt, wpool = _window_pool(w, w_sink, w_recent)
    q = workloads.bits(w.q)
    out = oracle.decode_windowed(pool, wpool, w.hkv, w.d, block, q, oracle.F16, w.block_table, wbt,
                                 w.seq_lens, w_sink, w_recent, w.sm_scale)
    g = w.hq // w.hkv
    rinv = np.eye(w.d) if block == 0 else np.kron(np.eye(w.d // block), scipy.linalg.hadamard(block)) / np.sqrt(block)
    qf = w.q.float().numpy().astype(np.float64)
    kin = w.k.to(torch.bfloat16).float().numpy().astype(np.float64)
    vin = w.v.to(torch.bfloat16).float().numpy().astype(np.float64)
    for b in range(w.batch):
        n = int(w.seq_lens[b])
        idx = np.nonzero(w.token_seq == b)[0]
        idx = idx[np.argsort(w.token_pos[idx])]
        for h in range(w.hq):
            kvh = h // g
            kk = _dequant_seq(w, pool, b, kvh, 0) @ rinv.T
            vv = _dequant_seq(w, pool, b, kvh, 1) @ rinv.T
            for t in range(n):
                if t < w_sink or t >= n - w_recent:
                    kk[t] = kin[idx[t], kvh]
                    vv[t] = vin[idx[t], kvh]
            p = scipy.special.softmax(w.sm_scale * kk @ qf[b, h])
            assert np.abs(out[b, h] - p @ vv).max() <= 1e-12 * max(1.0, np.abs(vv).max())


def test_windowed_absent_pages_leave_their_tokens_out():
    """Absent pages in either table (ids outside the INT4 pool or outside the
    window pool) drop their tokens: the row equals one scipy softmax over the
    hand-assembled keys and values of the remaining tokens, and a row whose
    every page is absent is zero."""
    block, w_sink, w_recent = 64, 4, 12
    w, pool = _tiny_case(seed=11, block=block, lens=[53, 40, 6])
    wbt, wpool = _window_pool(w, w_sink, w_recent)
    q = workloads.bits(w.q)
    bt = w.block_table.copy()
    wt = wbt.copy()
    n_win_pages = wpool.size // (w.hkv * oracle.bf16_slab_bytes(16, w.d))
    bt[0][1] = -1                      # INT4 tokens 16..31 of sequence 0
    wt[0][0] = n_win_pages + 2         # window positions 0..15: every window token of sequence 0
    bt[1][1] = w.num_pages             # INT4 tokens 16..27 of sequence 1 (28..39 are recent)
    bt[2][0] = -3                      # sequence 2 (6 tokens) lies in the window only ...
    wt[2][:] = -1                      # ... and its window pages are absent too
    out = oracle.decode_windowed(pool, wpool, w.hkv, w.d, block, q, oracle.F16, bt, wt,
                                 w.seq_lens, w_sink, w_recent, w.sm_scale)
    g = w.hq // w.hkv
    rinv = np.kron(np.eye(w.d // block), scipy.linalg.hadamard(block)) / np.sqrt(block)
    qf = w.q.float().numpy().astype(np.float64)
    kin = w.k.to(torch.bfloat16).float().numpy().astype(np.float64)
    vin = w.v.to(torch.bfloat16).float().numpy().astype(np.float64)
    for b in range(2):
        n = int(w.seq_lens[b])
        idx = np.nonzero(w.token_seq == b)[0]
        idx = idx[np.argsort(w.token_pos[idx])]
        for h in range(w.hq):
            kvh = h // g
            kk = _dequant_seq(w, pool, b, kvh, 0) @ rinv.T
            vv = _dequant_seq(w, pool, b, kvh, 1) @ rinv.T
            keep = []
            for t in range(n):
                windowed = t < w_sink or t >= n - w_recent
                if windowed:
                    kk[t] = kin[idx[t], kvh]
                    vv[t] = vin[idx[t], kvh]
                    pos = t if t < w_sink else w_sink + (t - w_sink) % w_recent
                    present = 0 <= wt[b][pos // 16] < n_win_pages
                else:
                    present = 0 <= bt[b][t // 16] < w.num_pages
                if present:
                    keep.append(t)
            keep = np.array(keep)
            assert 0 < len(keep) < n
            p = scipy.special.softmax(w.sm_scale * kk[keep] @ qf[b, h])
            assert np.abs(out[b, h] - p @ vv[keep]).max() <= 1e-12 * max(1.0, np.abs(vv).max())
    assert not out[2].any()


def test_windowed_ring_after_decode_steps():
    """Appending one token at a time into the ring keeps exactly the last
    w_recent tokens: the oracle then equals the brute force over the final
    length, though every ring slot was overwritten."""
    lens = np.array([30, 19])
    w, pool = _tiny_case(seed=9, block=16, lens=lens)
    w_sink, w_recent = 3, 5
    rng = np.random.default_rng(4)
    wbt, npages = workloads.window_layout(w.batch, w_sink, w_recent, rng)
    wpool = oracle.new_bf16_pool(npages, w.hkv, w.d)
    kb, vb = workloads.bits(w.k), workloads.bits(w.v)
    order = np.lexsort((w.token_seq, w.token_pos))      # by position, as decode steps append
    for i in order:
        # the sequence has token_pos + 1 tokens right after this append
        s = workloads.window_slots(wbt, w.token_seq[i:i + 1], w.token_pos[i:i + 1],
                                   np.full(w.batch, w.token_pos[i] + 1), w_sink, w_recent)
        oracle.append_bf16(wpool, npages, w.hkv, w.d, kb[i:i + 1], vb[i:i + 1], oracle.F16, s)
    ref_wbt, ref_pool = _window_pool(w, w_sink, w_recent, seed=4)
    q = workloads.bits(w.q)
    got = oracle.decode_windowed(pool, wpool, w.hkv, w.d, 16, q, oracle.F16, w.block_table, wbt,
                                 w.seq_lens, w_sink, w_recent, w.sm_scale)
    want = oracle.decode_windowed(pool, ref_pool, w.hkv, w.d, 16, q, oracle.F16, w.block_table, ref_wbt,
                                  w.seq_lens, w_sink, w_recent, w.sm_scale)
    assert np.array_equal(got, want)


def test_thread_count_does_not_change_results():
    """The oracle's threads split independent vectors and rows, so one thread
    and all of them give the same bytes and the same attention."""
    w = workloads.random_decode(71, batch=3, hq=8, hkv=2, d=64, block=32, seq_lens=[50, 1, 33])
    outs = []
    n = oracle.num_threads()
    try:
        for t in (1, n):
            oracle.set_num_threads(t)
            pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
            oracle.append_int4(pool, w.num_pages, w.hkv, w.d, 32, workloads.bits(w.k),
                               workloads.bits(w.v), oracle.BF16, w.slot_mapping.numpy())
            att = oracle.decode_int4(pool, w.hkv, w.d, 32, workloads.bits(w.q), oracle.BF16,
                                     w.block_table, w.seq_lens, w.sm_scale)
            outs.append((pool.copy(), att))
    finally:
        oracle.set_num_threads(n)
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])
