"""The benchmark's algorithmic byte counts agree with the stored layouts: the
bytes per stored vector bench.py charges equal the page slabs the oracle lays
out (CPU only)."""
import bench
import oracle


def setup_module(_):
    oracle.build(force=False)


def test_int4_vector_bytes_match_the_oracle_slab():
    for d in (64, 128):
        slab = oracle.int4_slab_bytes(16, d)        # 16 tokens x (K, V)
        assert bench.int4_bytes_per_vector(d) * 2 * 16 == slab


def test_decode_and_append_bytes():
    # two sequences of 16 and 17 tokens (1 + 2 pages), 8 KV heads, 32 q heads, d 128
    got = bench.decode_bytes([16, 17], 8, 32, 128, bench.int4_bytes_per_vector(128))
    want = 33 * 8 * 2 * 68 + 2 * 32 * 128 * (2 + 4) + 3 * 4 + 2 * 4
    assert got == want
    assert bench.append_bytes(10, 8, 128, 68) == 10 * 8 * 2 * 128 * 2 + 10 * 4 + 10 * 8 * 2 * 68
