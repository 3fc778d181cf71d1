"""Merging attention partials computed over disjoint key sets (test infrastructure).

Page 2 (section on technical optimisations, FA4 kernel) says the split count
``num_splits`` is chosen from batch size, TP size and KV length: the key range is cut
into parts, each part yields its own normalised output and log-sum-exp, and the parts
are merged. For parts s with outputs O_s and log-sum-exps lse_s over disjoint key sets
whose union is the visible set, the exact merge is

    M   = max_s lse_s
    w_s = exp(lse_s - M)            (a part with no key has lse_s = -inf and w_s = 0)
    out = sum_s w_s O_s / sum_s w_s
    lse = M + ln(sum_s w_s)

because exp(lse_s) O_s is that part's unnormalised sum of exp(logit) * v.
"""

import numpy as np


def combine_partials(o_parts, lse_parts):
    """Merge partials: o_parts [S][...][D], lse_parts [S][...] -> (out [...][D], lse [...])."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)
    if np.any(np.isneginf(M)):
        raise ValueError("every row needs at least one non-empty part")
    w = np.where(np.isneginf(lse_parts), 0.0, np.exp(lse_parts - M))
    total = w.sum(axis=0)
    out = (w[..., None] * np.where(np.isneginf(lse_parts)[..., None], 0.0, o_parts)).sum(axis=0)
    return out / total[..., None], M + np.log(total)
