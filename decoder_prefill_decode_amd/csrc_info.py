"""Launch-shape rules of the library that host-side accounting needs to mirror."""


def decode_splits(capacity: int) -> int:
    """Split count of decode attention for a KV window (attn_decode_splits in k_attn.hip)."""
    n = (capacity + 31) // 32
    return max(1, min(32, n))


def partial_stride(head_dim: int) -> int:
    """Floats per (query head, split) partial row of decode attention: o[d], m, l, pad."""
    return head_dim + 4
