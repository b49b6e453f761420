"""Launch-shape rules of the library that host-side accounting needs to mirror."""

BAND = 64         # decode positions per split plan (kDecBand)
MAX_SPLITS = 32   # splits of the decode attention (kDecMaxSplits)
UNIT = 16         # slots a block scores per step (kDecWaves * 4)


def decode_plan(capacity: int, t: int, cap: int = MAX_SPLITS):
    """(nsplit, chunk) of the decode attention at position t (attn_decode_plan in k_attn.hip): the
    slots [0, tb) of t's band of 64 positions, tb its end (at most the capacity), in up to `cap`
    splits of a multiple of 16 slots."""
    band = max(t, 0) // BAND
    tb = max(1, min(capacity, (band + 1) * BAND))
    chunk = UNIT * (-(-tb // (UNIT * cap)))
    return -(-tb // chunk), chunk


def partial_stride(head_dim: int) -> int:
    """Floats per (query head, split) partial row of decode attention: o[d], m, l, pad."""
    return head_dim + 4
