"""Benchmark of the INT4 KV-cache hot path (placeholder: accounting only)."""


def overhead_bits(bits: int, group: int) -> float:
    """Bits of a per-group parameter averaged over the numbers of the group."""
    return bits / group


def int4_bytes_per_vector(d: int) -> int:
    """Stored bytes of one (token, KV head, K|V) vector: D nibbles + fp16 scale + fp16 zero."""
    return d // 2 + 4
