"""Pins of the oracle's key scale search (BitDecoding-FP4 Abstract: scale
search under token-wise scaling) and of the hybrid symmetric/asymmetric group
quantizer (InnerQ Abstract and Figure 3), against worked closed forms, exact
arithmetic, brute force over the candidate grid and invariants -- nothing
here retypes the oracle's steps."""

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
    return float(np.uint16(h & 0x7FFF).view(np.float16)) * (-1.0 if h & 0x8000 else 1.0)


def _decode(codes, scale, zero):
    """Decoded values in fp64 (code * |scale| + zero, exact)."""
    return codes.astype(np.float64) * abs(_f16(scale)) + _f16(zero)


def _outlier_vectors(rng, n, d=128, factor=12.0):
    ys = rng.standard_normal((n, d)).astype(np.float32)
    for y in ys:
        y[rng.integers(0, d, 2)] *= factor
    return ys


# ---------------------------------------------------------------- the grid SSE

def test_grid_exponent_against_numpy_frexp():
    for a in (1.0, 0.75, 3.0, 1e-3, 6.0e4, 2.0 ** -30, 0.5):
        assert oracle.grid_exponent(a) == 20 - int(np.frexp(np.float32(a))[1])


def test_grid_sse_worked_errors():
    """y = decoded + m_i 2^-k with decoded exact and m_i small integers: the
    SSE is sum m_i^2 exactly, in any element order."""
    k = 20
    codes = np.array([0, 3, 15, 7, 8, 1], np.uint8)
    scale = int(np.float16(0.125).view(np.uint16))
    zero = int(np.float16(-1.0).view(np.uint16))
    m = np.array([0, 1, -2, 3, -5, 7])
    y = (_decode(codes, scale, zero) + m * 2.0 ** -k).astype(np.float32)
    assert np.array_equal(y.astype(np.float64), _decode(codes, scale, zero) + m * 2.0 ** -k)
    assert oracle.grid_sse(y, codes, scale, zero, k) == int((m * m).sum())
    perm = np.array([5, 2, 0, 4, 1, 3])
    assert oracle.grid_sse(y[perm], codes[perm], scale, zero, k) == int((m * m).sum())
    # half-integer errors on the grid round to even: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2
    h = np.array([0.5, 1.5, 2.5, -0.5, -1.5, 0.0])
    y2 = (_decode(codes, scale, zero) + h * 2.0 ** -k).astype(np.float32)
    assert oracle.grid_sse(y2, codes, scale, zero, k) == 0 + 4 + 4 + 0 + 4 + 0


def test_grid_sse_bounds_the_exact_sse():
    """On the grid 2^-k each error is off by at most half a step, so the
    grid SSE times 4^-k and the exact fp64 SSE differ by at most
    sum (|e_i| + 2^-k-1) 2^-k."""
    rng = np.random.default_rng(3)
    for y in _outlier_vectors(rng, 50):
        codes, s, z = oracle.quantize(y)
        k = oracle.grid_exponent(float(np.abs(y).max()))
        e = y.astype(np.float64) - _decode(codes, s, z)
        exact = float((e * e).sum())
        grid = oracle.grid_sse(y, codes, s, z, k) * 4.0 ** -k
        slack = float(((np.abs(e) + 2.0 ** (-k - 1)) * 2.0 ** -k).sum())
        assert abs(grid - exact) <= slack


# ---------------------------------------------------------------- scale search

def test_search_on_an_exact_grid_keeps_the_plain_quantizer():
    """A key vector that the plain quantizer reproduces exactly (zero -1,
    scale 1/8, codes spanning 0..15) has SSE 0 at j = 0, and ties go to the
    smallest j: the search returns the plain result."""
    rng = np.random.default_rng(4)
    k = rng.integers(0, 16, 128)
    k[:2] = [0, 15]
    y = (-1.0 + 0.125 * k).astype(np.float32)
    codes, s, z, j = oracle.quantize_search(y)
    assert j == 0
    assert np.array_equal(codes, k) and _f16(s) == 0.125 and _f16(z) == -1.0


def test_search_ties_go_to_the_least_clipping():
    """A zero key vector: every candidate is the same (range 0, SSE 0), and
    the tie goes to j = 0."""
    codes, s, z, j = oracle.quantize_search(np.zeros(128, np.float32))
    assert j == 0 and s == 0 and z == 0 and not codes.any()


def _candidate(y, j):
    """Candidate j built by another route: the plain quantizer applied to y
    clipped to [mn alpha_j, mx alpha_j] has exactly that range (mn < 0 < mx),
    so it yields candidate j's zero and scale; and because the codes are a
    monotone function of y clamped to [0, 15], the clipped vector's codes are
    the codes of y itself (checked: the range ends take codes 0 and 15)."""
    alpha = np.float32((16 - j) / 16)
    lo, hi = np.float32(y.min() * alpha), np.float32(y.max() * alpha)
    codes, s, z = oracle.quantize(np.clip(y, lo, hi))
    ends, _, _ = oracle.quantize(np.array([lo, hi] + [0.0] * 6, np.float32))
    assert ends[0] == 0 and ends[1] == 15
    return codes, s, z


def test_search_picks_the_argmin_of_its_grid_by_brute_force():
    rng = np.random.default_rng(5)
    for y in _outlier_vectors(rng, 40):
        assert y.min() < 0 < y.max()
        k = oracle.grid_exponent(float(np.abs(y).max()))
        cands = [_candidate(y, j) for j in range(8)]
        sse = [oracle.grid_sse(y, c, s, z, k) for c, s, z in cands]
        codes, s, z, j = oracle.quantize_search(y)
        assert j == int(np.argmin(sse))                   # argmin, the first on a tie
        assert np.array_equal(codes, cands[j][0]) and (s, z) == cands[j][1:]


def test_search_never_worse_than_plain_and_clips_outliers():
    """The chosen candidate's exact squared error is no larger than the plain
    quantizer's (up to the grid's rounding), its scale no larger, and on keys
    with x12 outlier channels it clips most vectors and lowers the total
    error."""
    rng = np.random.default_rng(6)
    tot_plain = tot_search = 0.0
    clipped = 0
    for y in _outlier_vectors(rng, 200):
        pc, ps, pz = oracle.quantize(y)
        sc, ss, sz, j = oracle.quantize_search(y)
        k = oracle.grid_exponent(float(np.abs(y).max()))
        ep = float(((y - _decode(pc, ps, pz)) ** 2).sum())
        es = float(((y - _decode(sc, ss, sz)) ** 2).sum())
        assert es <= ep + 2 * 128 * 2.0 ** (-2 * k + 22)
        assert _f16(ss) <= _f16(ps)
        tot_plain += ep
        tot_search += es
        clipped += j > 0
    assert clipped > 100
    assert tot_search < 0.95 * tot_plain


def test_search_pool_keeps_values_plain():
    """append_int4_search writes the INT4 layout: every V byte and V sidecar
    equals the plain append's, and each K vector equals quantize_search of the
    rotated input (read through the documented layout)."""
    w = workloads.random_decode(41, batch=2, hq=8, hkv=2, d=128, block=64, seq_lens=[37, 20])
    kb, vb, sm = workloads.bits(w.k), workloads.bits(w.v), w.slot_mapping.numpy()
    plain = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
    oracle.append_int4(plain, w.num_pages, w.hkv, w.d, 64, kb, vb, oracle.BF16, sm)
    srch = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
    oracle.append_int4_search(srch, w.num_pages, w.hkv, w.d, 64, kb, vb, oracle.BF16, sm)
    slab = oracle.int4_slab_bytes(16, w.d)
    p, d = 16, w.d
    for page in range(w.num_pages):
        for h in range(w.hkv):
            base = (page * w.hkv + h) * slab
            v_codes = slice(base + p * d // 2, base + p * d)
            v_side = slice(base + p * d + 4 * p, base + p * d + 8 * p)
            assert np.array_equal(plain[v_codes], srch[v_codes])
            assert np.array_equal(plain[v_side], srch[v_side])
    kf = w.k.float().numpy()
    changed = 0
    for t in range(len(sm)):
        page, off = divmod(int(sm[t]), 16)
        for h in range(w.hkv):
            y = oracle.rotate(kf[t, h], 64)
            codes, s, z, j = oracle.quantize_search(y)
            base = (page * w.hkv + h) * slab
            raw = srch[base + off * d // 2: base + (off + 1) * d // 2]
            got = np.stack([raw & 15, raw >> 4], axis=1).reshape(-1)
            side = srch[base + p * d + 4 * off: base + p * d + 4 * off + 4].view(np.uint16)
            assert np.array_equal(got, codes) and int(side[0]) == s and int(side[1]) == z
            changed += j > 0
    assert changed > 0


# ---------------------------------------------------------------- hybrid mode

def test_hybrid_symmetric_grid_is_exact_and_marked():
    """Values (k - 8)/8 with k spanning 1..15 (so max |y| = 7/8): the
    symmetric candidate has scale 7/8 / 7 = 1/8 exactly and zero -1, and
    reproduces every value (SSE 0); the asymmetric one (scale fp16(14/8/15))
    does not, so the group is symmetric: codes k, the scale's sign bit set."""
    rng = np.random.default_rng(7)
    k = rng.integers(1, 16, 64)
    k[:2] = [1, 15]
    y = ((k - 8) / 8).astype(np.float32)
    codes, s, z, sym = oracle.quantize_hybrid(y)
    assert sym and s == (int(np.float16(0.125).view(np.uint16)) | 0x8000)
    assert _f16(z) == -1.0 and np.array_equal(codes, k)
    assert np.array_equal(_decode(codes, s, z), y.astype(np.float64))


def test_hybrid_asymmetric_grid_stays_asymmetric():
    """Values -1 + k/8 with k spanning 0..15 (an exact asymmetric grid whose
    zero point is not -8 times a scale that reaches max |y| = 1): asymmetric,
    exact, no sign bit."""
    rng = np.random.default_rng(8)
    k = rng.integers(0, 16, 32)
    k[:2] = [0, 15]
    y = (-1.0 + k / 8).astype(np.float32)
    codes, s, z, sym = oracle.quantize_hybrid(y)
    assert not sym and not (s & 0x8000)
    assert np.array_equal(codes, k) and np.array_equal(_decode(codes, s, z), y.astype(np.float64))


def test_hybrid_tie_goes_to_symmetric():
    """Values +-105/16 lie on both grids: symmetric scale 105/16 / 7 = 15/16
    with zero -7.5 (codes 1 and 15), asymmetric zero -105/16 with scale
    (105/8) / 15 = 7/8 (codes 0 and 15), all exact in fp16 -- both SSEs are
    0, and the tie goes to the symmetric mode (no zero point of its own)."""
    y = np.array([-105 / 16, 105 / 16] * 16, np.float32)
    ac, as_, az = oracle.quantize(y)
    assert _f16(as_) == 0.875 and _f16(az) == -105 / 16
    assert np.array_equal(_decode(ac, as_, az), y.astype(np.float64))
    codes, s, z, sym = oracle.quantize_hybrid(y)
    assert sym and abs(_f16(s)) == 15 / 16 and _f16(z) == -7.5
    assert np.array_equal(codes, np.array([1, 15] * 16))


@pytest.mark.parametrize("lo,hi", [(1.0, 2.0), (-3.0, -0.5)])
def test_hybrid_one_signed_groups_are_asymmetric(lo, hi):
    """All values of one sign: a grid through 0 wastes half its levels."""
    rng = np.random.default_rng(9)
    y = rng.uniform(lo, hi, 64).astype(np.float32)
    _, s, _, sym = oracle.quantize_hybrid(y)
    assert not sym and not (s & 0x8000)


def test_hybrid_zero_group():
    codes, s, z, sym = oracle.quantize_hybrid(np.zeros(32, np.float32))
    assert not sym and s == 0 and z == 0 and not codes.any()


def test_hybrid_rule_and_error_bound():
    """On Gaussian groups: the mode is the candidate with the smaller grid SSE
    (the plain quantizer is the asymmetric candidate), symmetric groups have
    zero point exactly -8 |scale|, and every element decodes within half a
    scale step (plus the clamp slack of an fp16-rounded scale)."""
    rng = np.random.default_rng(10)
    n_sym = 0
    for g in (32, 64):
        for _ in range(300):
            y = rng.standard_normal(g).astype(np.float32)
            codes, s, z, sym = oracle.quantize_hybrid(y)
            ac, as_, az = oracle.quantize(y)
            kk = oracle.grid_exponent(float(np.abs(y).max()))
            mine = oracle.grid_sse(y, codes, s, z, kk)
            asym = oracle.grid_sse(y, ac, as_, az, kk)
            if sym:
                n_sym += 1
                assert mine <= asym and _f16(z) == -8 * abs(_f16(s))
                assert abs(_f16(s)) == float(np.float16(np.float32(np.abs(y).max()) / np.float32(7)))
            else:
                assert (codes, s, z) == (codes, as_, az) and np.array_equal(codes, ac)
            err = np.abs(y - _decode(codes, s, z))
            assert err.max() <= abs(_f16(s)) * (0.5 + 2.0 ** -7)
    assert 0 < n_sym < 600


def test_hybrid_pool_layout_and_attention():
    """append_int4g_hybrid writes the grouped layout with the mode in each
    scale's sign bit; attention over it (decode_int4g) equals scipy softmax
    attention over rows decoded from the layout text with |scale|, rotated
    back with scipy's Hadamard."""
    w = workloads.random_decode(42, batch=2, hq=8, hkv=2, d=64, block=32, seq_lens=[41, 19])
    g = 32
    pool = oracle.new_int4g_pool(w.num_pages, w.hkv, w.d, g)
    oracle.append_int4g_hybrid(pool, w.num_pages, w.hkv, w.d, 32, g, workloads.bits(w.k),
                               workloads.bits(w.v), oracle.BF16, w.slot_mapping.numpy())
    slab = oracle.int4g_slab_bytes(16, w.d, g)
    p, d, ng = 16, w.d, w.d // g

    def row(page, h, off, kind):
        base = (page * w.hkv + h) * slab
        vals = np.empty(d)
        side = pool[base + p * d + kind * 4 * p * ng: base + p * d + (kind + 1) * 4 * p * ng].view(np.uint16)
        for c in range(d):
            if kind == 0:
                byte = pool[base + off * d // 2 + c // 2]
                code = (byte >> 4) if c % 2 else (byte & 15)
            else:
                n, j = c % (d // 8), c // (d // 8)
                byte = pool[base + p * d // 2 + (n * p + off) * 4 + j // 2]
                code = (byte >> 4) if j % 2 else (byte & 15)
            sc, ze = side[2 * (off * ng + c // g)], side[2 * (off * ng + c // g) + 1]
            vals[c] = code * abs(_f16(int(sc))) + _f16(int(ze))
        return vals

    n_sym = int((pool.reshape(-1, slab)[:, p * d:].view(np.uint16)[:, 0::2] & 0x8000).astype(bool).sum())
    assert n_sym > 0
    q = workloads.bits(w.q)
    out = oracle.decode_int4g(pool, w.hkv, w.d, 32, g, q, oracle.BF16, w.block_table, w.seq_lens, w.sm_scale)
    rinv = np.kron(np.eye(d // 32), scipy.linalg.hadamard(32)) / np.sqrt(32)
    qf = w.q.float().numpy().astype(np.float64)
    grp = w.hq // w.hkv
    for b in range(w.batch):
        n = int(w.seq_lens[b])
        for h in range(w.hq):
            kk = np.array([row(int(w.block_table[b, t // 16]), h // grp, t % 16, 0) for t in range(n)]) @ rinv.T
            vv = np.array([row(int(w.block_table[b, t // 16]), h // grp, t % 16, 1) for t in range(n)]) @ rinv.T
            pr = scipy.special.softmax(w.sm_scale * kk @ qf[b, h])
            assert np.abs(out[b, h] - pr @ vv).max() <= 1e-12 * max(1.0, np.abs(vv).max())


def test_hybrid_pool_total_error_no_larger_than_asymmetric():
    """Group by group the hybrid keeps the candidate with the smaller grid
    SSE, so over a pool its exact reconstruction error stays at (or, within
    the grid's rounding, below) the asymmetric pool's."""
    rng = np.random.default_rng(11)
    tot_h = tot_a = 0.0
    for _ in range(200):
        y = rng.standard_normal(64).astype(np.float32)
        hc, hs, hz, _ = oracle.quantize_hybrid(y)
        ac, as_, az = oracle.quantize(y)
        tot_h += float(((y - _decode(hc, hs, hz)) ** 2).sum())
        tot_a += float(((y - _decode(ac, as_, az)) ** 2).sum())
    assert tot_h <= tot_a * (1 + 1e-6)
