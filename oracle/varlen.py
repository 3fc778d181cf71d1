"""Attention with a different number of query rows per sequence (test infrastructure).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark use this
module; the product path never does.

Page 3 ("vLLM supports Reflection Beam", section on DFlash2 and adaptive verification)
describes a verifier that decides at every step which draft tokens are worth checking,
so that the sequences of one batch verify different numbers of tokens; page 2 ("vLLM
TML Inkling support", model architecture section) lets one forward step produce up to 9
tokens from chained MTP heads. Either way, sequence b brings its own n_b query rows.

Definition: the rows of all sequences are packed one after another, sequence b owning
rows cu_rows[b] .. cu_rows[b+1]-1 (n_b = cu_rows[b+1] - cu_rows[b], possibly 0). Its
rows are its last n_b positions, exactly as in a fixed-row call with n = n_b on that
sequence alone: row i sits at position L_b - n_b + i and attends causally (and within
the window) over the sequence's keys. So each sequence is that call, and the packed
result is the rows of those calls laid end to end.
"""

import numpy as np

from .attention import relative_attention


def relative_attention_varlen(q, cu_rows, k_cache, v_cache, page_table, seq_lens, bias, *,
                              window, dmax, softmax_scale, k_scale=None, v_scale=None,
                              batches=None, kv_heads=None):
    """Return (out [T][Hq][D], lse [T][Hq]) in float64 for packed rows q [T][Hq][D].

    ``cu_rows`` [B+1] is nondecreasing from 0 to at most T; rows past cu_rows[B], and the
    rows of sequences or KV heads left out of ``batches`` / ``kv_heads``, are NaN.
    """
    q = np.asarray(q)
    cu = [int(x) for x in cu_rows]
    B = len(cu) - 1
    if cu[0] != 0 or any(cu[b + 1] < cu[b] for b in range(B)) or cu[B] > q.shape[0]:
        raise ValueError("cu_rows must rise from 0 to at most the number of rows")
    T, Hq, D = q.shape
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    for b in (range(B) if batches is None else batches):
        n_b = cu[b + 1] - cu[b]
        if n_b == 0:
            continue
        o, s = relative_attention(q[cu[b]:cu[b + 1]][None], k_cache, v_cache,
                                  np.asarray(page_table)[b:b + 1],
                                  np.asarray(seq_lens)[b:b + 1], bias, n_query_rows=n_b,
                                  window=window, dmax=dmax, softmax_scale=softmax_scale,
                                  k_scale=k_scale, v_scale=v_scale, kv_heads=kv_heads)
        out[cu[b]:cu[b + 1]] = o[0]
        lse[cu[b]:cu[b + 1]] = s[0]
    return out, lse
