"""Benchmark (placeholder while the library is being built)."""


def kv_cache_bytes(kv_heads, head_dim, positions, bytes_per):
    """Bytes of one layer's K and V cache for one request: 2 (K and V) x heads x width x positions x bytes."""
    return 2 * kv_heads * head_dim * positions * bytes_per
