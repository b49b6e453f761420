"""Shared parity helpers of the GPU tests.

Every expected value and every tolerance here comes from the oracle (or is a
fixed gate); nothing is derived from the GPU's own output.

Greedy ids: fp32 workloads must reproduce the oracle's ids exactly. For bf16
workloads the oracle's result is fixed only up to its noise floor: rerun with
float32 BLAS sums instead of exact ones (every operand and rounding point
unchanged) and teacher-forced on the exact ids, its logits move by up to
`floor` at some step. A step whose exact top-2 margin is below that floor is a
near-tie that the arithmetic does not decide; at every other step the GPU,
teacher-forced on the oracle's ids, must pick the oracle's id, and a
free-running GPU sequence may first leave the oracle's only at a near-tie.
"""
import numpy as np

from oracle import decoder as od


def rel(a, b):
    """max |a - b| / max |b| (the gate's relative error)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def oracle_run(cfg, glob, layers, **kw):
    """The oracle's run plus, for bf16 workloads, its noise floor (ref['floor'];
    0 for fp32 workloads, whose ids are compared exactly)."""
    ref = od.run_decoder(cfg, glob, layers, keep_logits=True, **kw)
    ref["floor"] = 0.0
    if cfg.dtype == "bf16" and cfg.vocab > 0:
        p = od.run_decoder(cfg, glob, layers, keep_logits=True, prec=od.BF16_F32SUM, forced_ids=ref["ids"][:-1], **kw)
        ref["floor"] = max(float(np.abs(a - b).max())
                           for a, b in zip([ref["logits0"]] + ref["step_logits"], [p["logits0"]] + p["step_logits"]))
    return ref


def check_ids(label, free, forced, ref_ids, margins, floor):
    """Greedy-id gate (see the module docstring). free: GPU free-running ids;
    forced: GPU picks when fed the oracle's ids (forced[0] is the prefill's pick).
    Returns (free agreement, forced agreement, exempt steps, first divergence)."""
    ref_ids = [int(i) for i in ref_ids]
    n = len(ref_ids)
    exempt = {i for i in range(n) if margins[i] < floor}
    agree_free = sum(int(a == b) for a, b in zip(free, ref_ids))
    agree_forced = sum(int(a == b) for a, b in zip(forced, ref_ids))
    div = next((i for i in range(n) if free[i] != ref_ids[i]), None)
    flips = [i for i in range(n) if forced[i] != ref_ids[i]]
    print(f"{label}: free-running agreement {agree_free}/{n} (first divergence {div}), teacher-forced "
          f"agreement {agree_forced}/{n}, flips at {flips} with margins {[round(float(margins[i]), 5) for i in flips]}; "
          f"{len(exempt)}/{n} steps below the oracle's noise floor {floor:.3e}")
    bad = [i for i in flips if i not in exempt]
    assert not bad, f"{label}: teacher-forced mismatch at decided steps {bad} (margins {[margins[i] for i in bad]})"
    assert div is None or div in exempt, f"{label}: free-running divergence at decided step {div}"
    return agree_free, agree_forced, len(exempt), div
