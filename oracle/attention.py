"""Relative-position GQA decode/verify attention over a paged KV cache, in float64.

Test infrastructure: only the tests, the smoke check and the CPU-baseline leg of the
benchmark use this module; the product path never does.

What is computed (the plain definition, no blocking or fusion):

For sequence b with length L (the length counts the n new tokens, whose keys and
values are already in the cache), query row r in [0, n) sits at absolute position
``p = L - n + r``. Query head h reads KV head ``g = h div G`` with ``G = Hq / Hkv``
(grouped-query attention, page 2 model architecture section; page 1 model table:
48 query / 8 KV heads, head size 128). Key j is visible to row r when ``j <= p``
(causal; the n verify rows are causal among themselves, page 1 section on trying the
model: 7 draft tokens per step) and, in a sliding-window layer of width W (page 1
model table: 1,024), when ``p - j <= W - 1`` (W keys including the token itself).
W = 0 means a full-context layer.

    s_j = scale * (q . k_j) + B[h][min(p - j, Dmax)]          (page 2: a learned
                                                               relative term added to
                                                               the pre-softmax logits)
    out = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m),   m = max_j s_j
    lse = m + ln(sum_j exp(s_j - m))

Key j of sequence b lives in physical page ``page_table[b][j div S]`` at slot
``j mod S``; the cache is laid out ``[page][kv_head][slot][dim]``. For the FP8 cache
(page 2 roadmap, page 3 support section) the stored code is decoded to its E4M3 value
and multiplied by the float32 per-token-per-head scale ``scale[page][kv_head][slot]``.
"""

import numpy as np

from .formats import bf16_bits_to_f64, e4m3fn_codes_to_f64


def _decode(values):
    values = np.asarray(values)
    if values.dtype == np.uint16:
        return bf16_bits_to_f64(values)
    if values.dtype == np.uint8:
        return e4m3fn_codes_to_f64(values)
    if values.dtype in (np.float64, np.float32):
        return values.astype(np.float64)
    raise TypeError("unsupported stored dtype %s" % values.dtype)


def _gather_kv(cache, scale, page_table_row, keys, kv_head, page_size):
    """Values of keys ``keys`` for one KV head, as a float64 [len(keys)][D] array."""
    phys = np.asarray(page_table_row)[keys // page_size].astype(np.int64)
    slot = keys % page_size
    vals = _decode(cache[phys, kv_head, slot, :])
    if np.asarray(cache).dtype == np.uint8:
        if scale is None:
            raise ValueError("an FP8 cache needs its per-token-per-head scales")
        vals = vals * np.asarray(scale)[phys, kv_head, slot].astype(np.float64)[:, None]
    return vals


def _attend_group(q_rows, k_vals, v_vals, keys, positions, bias_rows, window, dmax,
                  softmax_scale, key_lo, key_hi):
    """Attention of one KV group.

    q_rows   float64 [n][G][D]   the G query heads of the group, for the n rows
    k_vals   float64 [nk][D]     keys ``keys`` of this KV head
    positions int64  [n]         absolute positions of the rows
    bias_rows float64 [G][Dmax+1]
    Keys outside [key_lo, key_hi) are left out (used for split partials).
    Returns out [n][G][D] and lse [n][G]; a row with no visible key gets out = 0
    and lse = -inf.
    """
    n, G, D = q_rows.shape
    logits = softmax_scale * (q_rows.reshape(n * G, D) @ k_vals.T).reshape(n, G, -1)
    dist = positions[:, None] - keys[None, :]                      # [n][nk]
    visible = dist >= 0
    if window > 0:
        visible &= dist <= window - 1
    visible &= (keys[None, :] >= key_lo) & (keys[None, :] < key_hi)
    idx = np.minimum(np.where(visible, dist, 0), dmax)            # never negative
    rel = bias_rows[:, idx]                                        # [G][n][nk]
    s = logits + np.transpose(rel, (1, 0, 2))                      # [n][G][nk]
    s = np.where(visible[:, None, :], s, -np.inf)
    any_visible = visible.any(axis=-1)                             # [n]
    m = np.where(any_visible[:, None], s.max(axis=-1, initial=-np.inf), 0.0)
    w = np.exp(s - m[..., None])
    l = w.sum(axis=-1)
    out = np.zeros((n, G, D))
    lse = np.full((n, G), -np.inf)
    ok = any_visible
    if ok.any():
        out[ok] = (w[ok] @ v_vals) / l[ok][..., None]
        lse[ok] = m[ok] + np.log(l[ok])
    return out, lse


def partial_attention(q, k_cache, v_cache, page_table, seq_lens, bias, *, n_query_rows,
                      window, dmax, softmax_scale, k_scale=None, v_scale=None,
                      key_lo=0, key_hi=None, batches=None, kv_heads=None):
    """Attention restricted to keys in [key_lo, key_hi) (same for every sequence).

    Returns (out, lse) like ``relative_attention``; rows with no visible key in the
    range get out = 0 and lse = -inf. Entries outside the requested ``batches`` /
    ``kv_heads`` subsets are NaN.
    """
    qv = _decode(q)
    B, n, Hq, D = qv.shape
    if n != n_query_rows:
        raise ValueError("q has %d rows per sequence, expected %d" % (n, n_query_rows))
    Hkv = np.asarray(k_cache).shape[1]
    page_size = np.asarray(k_cache).shape[2]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    bias64 = np.asarray(bias, dtype=np.float64)
    if bias64.shape != (Hq, dmax + 1):
        raise ValueError("bias must be [Hq][dmax+1]")
    seq_lens = np.asarray(seq_lens).astype(np.int64)
    page_table = np.asarray(page_table)
    out = np.full((B, n, Hq, D), np.nan)
    lse = np.full((B, n, Hq), np.nan)
    for b in (range(B) if batches is None else batches):
        L = int(seq_lens[b])
        if not n <= L:
            raise ValueError("seq_len %d is shorter than the %d query rows" % (L, n))
        positions = L - n + np.arange(n, dtype=np.int64)
        lo = 0 if window == 0 else max(0, L - n + 1 - window)
        keys = np.arange(lo, L, dtype=np.int64)
        hi = L if key_hi is None else key_hi
        for g in (range(Hkv) if kv_heads is None else kv_heads):
            kv = _gather_kv(k_cache, k_scale, page_table[b], keys, g, page_size)
            vv = _gather_kv(v_cache, v_scale, page_table[b], keys, g, page_size)
            heads = slice(g * G, (g + 1) * G)
            o, s = _attend_group(qv[b, :, heads, :], kv, vv, keys, positions,
                                 bias64[heads], window, dmax, softmax_scale, key_lo, hi)
            out[b, :, heads, :] = o
            lse[b, :, heads] = s
    return out, lse


def relative_attention(q, k_cache, v_cache, page_table, seq_lens, bias, *, n_query_rows,
                       window, dmax, softmax_scale, k_scale=None, v_scale=None,
                       batches=None, kv_heads=None):
    """Return (out, lse) in float64 for every sequence, query row and query head.

    q           [B][n][Hq][D]       bf16 codes (uint16) or float64 values
    k_cache     [P][Hkv][S][D]      bf16 codes (uint16), E4M3 codes (uint8) or float64
    v_cache     same as k_cache
    k_scale     [P][Hkv][S] float32 per-token-per-head scales (E4M3 caches only)
    v_scale     same
    page_table  [B][max_pages]      physical page of each logical page
    seq_lens    [B]                 sequence lengths, including the n query rows
    bias        [Hq][dmax+1]        relative-position table
    out         [B][n][Hq][D] float64;  lse [B][n][Hq] float64 (natural log)

    ``batches`` / ``kv_heads`` restrict the work to a sample; the other entries are NaN.
    """
    return partial_attention(q, k_cache, v_cache, page_table, seq_lens, bias,
                             n_query_rows=n_query_rows, window=window, dmax=dmax,
                             softmax_scale=softmax_scale, k_scale=k_scale,
                             v_scale=v_scale, batches=batches, kv_heads=kv_heads)
