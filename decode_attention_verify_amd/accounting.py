"""Algorithmic bytes and flops of one decode/verify attention call.

Every byte the method must move is counted once: the visible keys and values of each
KV head (plus their per-token scales in the FP8 cache), the bias entries at the
distances that some query reaches, the page-table entries and lengths read, the
queries, and the outputs (bf16 out and fp32 log-sum-exp). Split partials are an
implementation detail and are not algorithmic.

Flops: 4*D per (row, query head, visible key): 2*D for q.k and 2*D for p*v.
"""

from dataclasses import dataclass


@dataclass
class Traffic:
    kv: int
    scales: int
    bias: int
    q: int
    out: int
    lse: int
    page_table: int
    seq_lens: int
    flops: int
    visible_keys: int     # sum over sequences of keys visible to at least one row

    @property
    def total(self):
        return (self.kv + self.scales + self.bias + self.q + self.out + self.lse
                + self.page_table + self.seq_lens)


def visible_span(L, n, window):
    """Number of keys visible to at least one of the n rows of a sequence of length L."""
    if window == 0:
        return L
    return min(L, window + n - 1)


def rows_keys(L, n, window):
    """Sum over the n rows of the keys each row sees."""
    total = 0
    for r in range(n):
        p = L - n + r
        total += (p + 1) if window == 0 else min(window, p + 1)
    return total


def traffic(seq_lens, *, n_rows, num_q_heads, num_kv_heads, head_dim, window, dmax,
            page_size, kv_bytes_per_elem, with_lse=True, rows_per_seq=None):
    """``rows_per_seq``: each sequence's own row count (default n_rows for all)."""
    seq_lens = [int(x) for x in seq_lens]
    rows = [n_rows] * len(seq_lens) if rows_per_seq is None else [int(x) for x in rows_per_seq]
    live = [(L, n) for L, n in zip(seq_lens, rows) if n > 0]
    spans = [visible_span(L, n, window) for L, n in live]
    keys = sum(spans)
    kv = keys * num_kv_heads * head_dim * 2 * kv_bytes_per_elem
    scales = keys * num_kv_heads * 2 * 4 if kv_bytes_per_elem == 1 else 0
    if live:
        max_dist = max(((window - 1) if window > 0 else (L - 1)) for L, _ in live)
        max_dist = min(max_dist, max(L for L, _ in live) - 1)
        distinct = min(max_dist, dmax) + 1
    else:
        distinct = 0
    bias = num_q_heads * 4 * distinct
    total_rows = sum(rows)
    q = total_rows * num_q_heads * head_dim * 2
    out = q
    lse = total_rows * num_q_heads * 4 if with_lse else 0
    pages = 0
    for (L, _), s in zip(live, spans):
        lo = L - s
        pages += (L - 1) // page_size - lo // page_size + 1
    flops = sum(rows_keys(L, n, window) for L, n in live) * num_q_heads * 4 * head_dim
    cu = 4 * (len(seq_lens) + 1) if rows_per_seq is not None else 0
    return Traffic(kv=kv, scales=scales, bias=bias, q=q, out=out, lse=lse,
                   page_table=pages * 4 + cu, seq_lens=len(seq_lens) * 4, flops=flops,
                   visible_keys=keys)


def kv_bytes_per_token_per_layer(num_kv_heads, head_dim, kv_bytes_per_elem):
    """Bytes of K and V that one token adds to one attention layer's cache."""
    return 2 * num_kv_heads * head_dim * kv_bytes_per_elem


def append_traffic(seq_lens, *, n_rows, num_kv_heads, head_dim, page_size, kv_bytes_per_elem):
    """Algorithmic bytes of writing each sequence's n newest tokens into the cache: the
    new K and V rows read (bf16), the cache rows written (bf16, or E4M3 codes plus one
    fp32 scale per row), and the lengths and page-table entries read."""
    seq_lens = [int(x) for x in seq_lens]
    B = len(seq_lens)
    rows = B * n_rows * num_kv_heads * 2                     # K and V
    read = rows * head_dim * 2
    write = rows * head_dim * kv_bytes_per_elem + (rows * 4 if kv_bytes_per_elem == 1 else 0)
    pages = sum((L - 1) // page_size - (L - n_rows) // page_size + 1 for L in seq_lens)
    return read + write + pages * 4 + B * 4
