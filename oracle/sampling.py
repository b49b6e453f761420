"""Oracle for the next-token sampler: repetition penalty, temperature, top-k,
top-p, softmax and a draw.

TEST INFRASTRUCTURE: imported only by tests/ and bench.py's cpu_baseline leg.
Shares no code with the HIP path.

Sources (page title, section):
  [MNN]    MNN llm_demo Omni article (hmyw.cn news 148174), §4.1: the logits are
           divided by the temperature, cut to the top-k values (values below the
           k-th largest become -inf), cut by top-p (sorted by probability, the
           tokens after the cumulative probability passes the threshold become
           -inf), then softmax and a draw (or the maximum); a repeat penalty acts
           on tokens already in the context during the same post-processing.
  [HyOCR15] HunyuanOCR v1.5 ncnn port, §3.6 (generation options: temperature,
           top_p / top_k, repetition penalty, sample or not) and §4 (unit tests
           cover the repetition penalty).

Readings where the pages are silent (listed with the design notes):
  * The penalty comes first and is the usual one for logits of either sign: a
    context token's logit x becomes x / r if x > 0, else x * r (r >= 1); each
    distinct context id is penalised once.
  * Ties: top-k keeps every value equal to the k-th largest (the page removes
    only smaller values); the top-p order is probability descending, then id
    ascending, and the token whose addition reaches the threshold is kept.
  * The draw is the inverse CDF of the kept tokens in that same order, with the
    uniform number u in [0, 1) passed in by the caller (the random draw is an
    input, so both sides see the same one): the first token whose cumulative
    probability exceeds u times the kept total.
"""
import numpy as np


def penalize(logits, context_ids, penalty):
    """Repetition penalty on the distinct ids of the context (reading above)."""
    x = np.asarray(logits, np.float64).copy()
    if penalty != 1.0 and len(context_ids):
        ids = np.unique(np.asarray(context_ids, np.int64))
        v = x[ids]
        x[ids] = np.where(v > 0, v / penalty, v * penalty)
    return x


def sample_token(logits, context_ids, temperature, top_k, top_p, penalty, u):
    """One sampled id, in the steps and order of [MNN] §4.1 (float64).

    Returns (id, info): info holds the decision margins a lower-precision
    implementation could fall on the other side of: the gap between the k-th
    and the (k+1)-th value, the distance of the top-p cumulative sums from the
    threshold, and the distance of u * total from the nearest CDF boundary (all
    relative to the kept total where they are probabilities).
    """
    x = np.asarray(logits, np.float64)
    if not np.all(np.isfinite(x)):
        raise FloatingPointError("non-finite logits")
    V = x.size
    x = penalize(x, context_ids, penalty) / temperature
    info = {}
    keep = np.ones(V, bool)
    if 0 < top_k < V:
        srt = np.sort(x)[::-1]
        kth = srt[top_k - 1]
        keep &= x >= kth
        nxt = srt[top_k:]
        below = nxt[nxt < kth]
        info["topk_gap"] = float(kth - below[0]) if below.size else np.inf
    # order: probability descending, id ascending
    idx = np.nonzero(keep)[0]
    order = idx[np.lexsort((idx, -x[idx]))]
    p = np.exp(x[order] - x[order[0]])
    Z = p.sum()
    if 0 < top_p < 1:
        before = np.concatenate([[0.0], np.cumsum(p)[:-1]])  # cumulative before each token
        kept = before < top_p * Z
        info["topp_margin"] = float(np.min(np.abs(before[1:] - top_p * Z)) / Z) if p.size > 1 else np.inf
        order, p = order[kept], p[kept]
    total = p.sum()
    cdf = np.cumsum(p)
    r = int(np.searchsorted(cdf, u * total, side="right"))
    r = min(r, order.size - 1)
    info["cdf_margin"] = float(np.min(np.abs(cdf[:-1] - u * total)) / total) if p.size > 1 else np.inf
    info["kept"] = int(order.size)
    info["probs"] = (order, p / total)
    return int(order[r]), info
