"""Launch-shape rules of the library that host-side accounting needs to mirror."""


def decode_splits(capacity: int) -> int:
    """Split count of decode attention for a KV window (attn_decode_splits in k_attn.hip)."""
    n = (capacity + 63) // 64
    return max(1, min(32, n))
