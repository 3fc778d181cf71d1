"""Writing new tokens' keys and values into the paged cache (test infrastructure).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark use this
module; the product path never does.

This is the step just before the attention: the n tokens that a decode or verify step
adds to each sequence get their K and V written into the cache pages that the
attention then reads. Page 3 ("vLLM supports Reflection Beam", section on speeding up
the implementation) speaks of a fused KV-cache update, and page 2's roadmap and page
3's support section of an FP8 KV cache.

Sequence b holds L_b tokens after the step; its new token r in [0, n) sits at position
t = L_b - n + r, in slot t mod S of physical page page_table[b][t div S].

For an E4M3 cache, each (token, KV head) vector x of head_dim values is stored as
codes c_d = E4M3(clamp(x_d / s, -448, 448)) with the fp32 scale s = max_d |x_d| / 448
(s = 1 when every x_d is 0), where E4M3(.) rounds to the nearest code, ties to the even
code. A code is an integer that floating point decides, so the quotients are taken in
float32, the precision the kernel computes them in: s = fp32(max |x|) / fp32(448) and
x_d / s, each correctly rounded. The rounding to E4M3 itself is exact arithmetic on
those float32 values.
"""

import numpy as np

from .formats import bf16_bits_to_f64

E4M3_MAX = 448.0


def e4m3fn_encode(values):
    """Round float values (any finite magnitude <= 448) to OCP E4M3 codes (uint8),
    to nearest with ties to even; from the format's definition (1 sign bit, 4
    exponent bits with bias 7, 3 fraction bits; subnormals 2**-6 * m/8)."""
    v = np.asarray(values, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("E4M3 encoding of non-finite values")
    if np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("magnitudes above 448 must be clamped first")
    sign = (np.signbit(v)).astype(np.uint8) << 7
    a = np.abs(v)
    # exponent of the binade holding a, with the subnormal binade folded into e = -6
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    # guard against log2 rounding at binade edges: make 2**e <= a < 2**(e+1) hold
    e = np.where((a > 0) & (np.exp2(e) > a) & (e > -6), e - 1, e)
    e = np.where((a > 0) & (np.exp2(e + 1) <= a), e + 1, e)
    quantum = np.exp2(e - 3)                       # 3 fraction bits
    k = a / quantum                                # exact: power-of-two scaling
    kr = np.floor(k)
    frac = k - kr
    kr = np.where((frac > 0.5) | ((frac == 0.5) & (np.fmod(kr, 2) == 1)), kr + 1, kr)
    mag = kr * quantum                             # the rounded magnitude
    out = np.zeros(a.shape, dtype=np.uint8)
    nz = mag > 0
    # re-derive the fields of the rounded value (rounding may move it up one binade)
    em = np.floor(np.log2(np.where(nz, mag, 1.0)))
    normal = nz & (em >= -6)
    exp_field = np.where(normal, em + 7, 0).astype(np.int64)
    frac_field = np.where(normal, mag / np.exp2(em) * 8 - 8, mag / 2.0 ** -9).astype(np.int64)
    code = (exp_field << 3) | frac_field
    out[nz] = code[nz].astype(np.uint8)
    return out | sign


def quantise_rows_e4m3(x_bits):
    """bf16 codes [..][D] -> (E4M3 codes [..][D] uint8, fp32 scales [..]), in float32."""
    x = bf16_bits_to_f64(x_bits).astype(np.float32)          # bf16 -> fp32 is exact
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)             # one correctly rounded quotient
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3fn_encode(y), scale


def append_kv(k_new, v_new, page_table, seq_lens, k_cache, v_cache, k_scale=None,
              v_scale=None):
    """Return copies of the caches (and scales) with the new tokens written.

    k_new, v_new  bf16 codes (uint16) [B][n][Hkv][D]
    k_cache ...   bf16 codes (uint16) or E4M3 codes (uint8) [P][Hkv][S][D]
    k_scale ...   fp32 [P][Hkv][S] for the E4M3 cache
    """
    k_new = np.asarray(k_new)
    v_new = np.asarray(v_new)
    B, n, Hkv, D = k_new.shape
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    fp8 = kc.dtype == np.uint8
    ks = None if k_scale is None else np.array(k_scale, copy=True)
    vs = None if v_scale is None else np.array(v_scale, copy=True)
    if fp8 and (ks is None or vs is None):
        raise ValueError("an E4M3 cache needs its scales")
    S = kc.shape[2]
    for b in range(B):
        L = int(seq_lens[b])
        if L < n:
            raise ValueError("sequence %d is shorter than its %d new tokens" % (b, n))
        for r in range(n):
            t = L - n + r
            page = int(page_table[b][t // S])
            slot = t % S
            for src, cache, scales in ((k_new, kc, ks), (v_new, vc, vs)):
                row = src[b, r]                                  # [Hkv][D] bf16 codes
                if fp8:
                    codes, sc = quantise_rows_e4m3(row)
                    cache[page, :, slot, :] = codes
                    scales[page, :, slot] = sc
                else:
                    cache[page, :, slot, :] = row
    return kc, vc, ks, vs
