"""Pure-Python brute force of relative-position GQA attention (test infrastructure).

The same definition as ``oracle.attention`` (page 2, model architecture section: a
learned relative term added to the pre-softmax logits; page 1 model table: GQA heads
and the sliding window), written a second time as explicit loops over every
(sequence, row, head, key, dim) with Python floats, for tiny inputs only. It reads a
contiguous cache ``[B][Hkv][L][D]`` of already-decoded values, so it shares no paging
or decoding step with the vectorised oracle.
"""

import math


def bruteforce_attention(q, k, v, seq_lens, bias, *, window, dmax, softmax_scale):
    """q [B][n][Hq][D], k/v [B][Hkv][Lmax][D] nested sequences of floats.

    Returns (out [B][n][Hq][D], lse [B][n][Hq]) as nested lists.
    """
    B = len(q)
    n = len(q[0])
    Hq = len(q[0][0])
    D = len(q[0][0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    out = [[[[0.0] * D for _ in range(Hq)] for _ in range(n)] for _ in range(B)]
    lse = [[[0.0] * Hq for _ in range(n)] for _ in range(B)]
    for b in range(B):
        L = int(seq_lens[b])
        for r in range(n):
            i = L - n + r                      # absolute position of this query row
            for h in range(Hq):
                g = h // G
                logits = []
                for j in range(L):
                    if j > i:
                        continue               # causal
                    if window > 0 and i - j >= window:
                        continue               # outside the window of W keys
                    dot = 0.0
                    for d in range(D):
                        dot += float(q[b][r][h][d]) * float(k[b][g][j][d])
                    rel = float(bias[h][min(i - j, dmax)])
                    logits.append((j, softmax_scale * dot + rel))
                m = max(s for _, s in logits)
                weights = [(j, math.exp(s - m)) for j, s in logits]
                total = sum(w for _, w in weights)
                for d in range(D):
                    acc = 0.0
                    for j, w in weights:
                        acc += w * float(v[b][g][j][d])
                    out[b][r][h][d] = acc / total
                lse[b][r][h] = m + math.log(total)
    return out, lse
