"""The KV-cache append on the GPU (through the C ABI) against the oracle.

Byte work, so the bar is bit-exact: every cache byte and every fp32 scale must equal
the oracle's, including the bytes the append must leave alone (NaN-poisoned slots,
other sequences' pages). The E4M3 rounding is checked exhaustively: rows whose largest
magnitude is 448 have scale 1, so their other elements reach the encoder unchanged,
and together they cover every bf16 value in [-448, 448].
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from decode_attention_verify_amd import binding, synth
from tests.parity import compare, oracle_of, run_hip, say

pytestmark = pytest.mark.gpu


def small(base, **kw):
    return dataclasses.replace(synth.spec(base), **kw)


def _new_rows(B, n, Hkv, D, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn((B, n, Hkv, D), generator=g).to(torch.bfloat16),
            torch.randn((B, n, Hkv, D), generator=g).to(torch.bfloat16))


def _as_codes(t):
    return t.view(torch.uint16 if t.dtype == torch.bfloat16 else torch.uint8).cpu().numpy()


def _from_codes(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(a)


def _oracle_append(case, k_new, v_new):
    return oracle.append_kv(
        _as_codes(k_new), _as_codes(v_new), case.page_table.numpy(), case.seq_lens.numpy(),
        _as_codes(case.k_cache), _as_codes(case.v_cache),
        None if case.k_scale is None else case.k_scale.numpy(),
        None if case.v_scale is None else case.v_scale.numpy())


def _same_bits(got, want, what):
    g = got.cpu().numpy() if isinstance(got, torch.Tensor) else got
    if g.dtype == np.float32:
        g, want = g.view(np.uint32), want.view(np.uint32)
    bad = np.argwhere(g != want)
    assert bad.size == 0, "%s: %d elements differ, first at %s" % (what, len(bad),
                                                                 bad[:4].tolist())


def _append_both(case, k_new, v_new, seq_lens=None, flags=True):
    """Run the GPU append on copies of the case's cache and scales."""
    prob = binding.problem_from_case(case)
    dev = "cuda"
    kc, vc = case.k_cache.clone().to(dev), case.v_cache.clone().to(dev)
    ks = None if case.k_scale is None else case.k_scale.clone().to(dev)
    vs = None if case.v_scale is None else case.v_scale.clone().to(dev)
    lens = case.seq_lens if seq_lens is None else seq_lens
    fl = torch.zeros(1, dtype=torch.int32, device=dev) if flags else None
    binding.rattn_append_kv(prob, k_new.to(dev), v_new.to(dev), case.page_table.to(dev),
                            lens.to(dev), kc, vc, ks, vs, fl)
    torch.cuda.synchronize()
    return kc, vc, ks, vs, (None if fl is None else int(fl.item())), prob


@pytest.mark.parametrize("fmt,page_size,n", [(synth.KV_BF16, 16, 1), (synth.KV_BF16, 16, 8),
                                             (synth.KV_BF16, 64, 9), (synth.KV_FP8, 16, 1),
                                             (synth.KV_FP8, 64, 8), (synth.KV_FP8, 256, 3)])
def test_append_matches_oracle_bytes(fmt, page_size, n):
    sp = small("full_100k", batch=5, n_rows=n, kv_format=fmt, page_size=page_size,
               seq_len=("uniform", n, 900), dmax=1000, name="append")
    case = synth.make_case(sp, seed=page_size + n)
    k_new, v_new = _new_rows(sp.batch, n, sp.num_kv_heads, sp.head_dim, seed=n)
    say("append %s page=%d n=%d lens=%s" % (fmt, page_size, n, case.seq_lens.tolist()))
    kc, vc, ks, vs, flags, _ = _append_both(case, k_new, v_new)
    assert flags == 0
    ok, ov, oks, ovs = _oracle_append(case, k_new, v_new)
    _same_bits(_as_codes(kc), ok, "K cache")
    _same_bits(_as_codes(vc), ov, "V cache")
    if fmt == synth.KV_FP8:
        # as bit patterns: the slots nothing writes hold NaN
        _same_bits(ks, oks, "K scales")
        _same_bits(vs, ovs, "V scales")


def test_e4m3_rounding_exhaustive():
    # every finite bf16 value with magnitude <= 448, 127 per row beside one 448 (scale 1)
    codes = np.arange(1 << 16, dtype=np.uint16)
    vals = oracle.bf16_bits_to_f64(codes)
    keep = codes[np.isfinite(vals) & (np.abs(vals) <= 448)]
    per_row = 127
    rows = -(-keep.size // per_row)
    Hkv = 8
    B = -(-rows // Hkv)
    data = np.zeros((B * Hkv, 128), dtype=np.uint16)
    flat = np.concatenate([keep, np.zeros(rows * per_row - keep.size, dtype=np.uint16)])
    data[:rows, 1:] = flat.reshape(rows, per_row)
    data[:, 0] = 0x43E0                                   # bf16 448.0
    sp = small("full_100k", batch=B, n_rows=1, num_q_heads=Hkv, num_kv_heads=Hkv,
               kv_format=synth.KV_FP8, page_size=16, seq_len=1, dmax=10, name="e4m3")
    case = synth.make_case(sp, seed=0)
    k_new = torch.from_numpy(data.reshape(B, 1, Hkv, 128).astype(np.int16)).view(torch.bfloat16)
    kc, vc, ks, vs, flags, _ = _append_both(case, k_new, k_new)
    assert flags == 0
    ok, ov, oks, ovs = _oracle_append(case, k_new, k_new)
    _same_bits(_as_codes(kc), ok, "E4M3 codes")
    _same_bits(ks, oks, "scales")
    pages = case.page_table[:, 0].numpy()
    assert np.all(ks.cpu().numpy()[pages, :, 0] == 1.0)     # the premise: scale 1 per row


@pytest.mark.parametrize("fmt", [synth.KV_BF16, synth.KV_FP8])
def test_append_then_decode(fmt):
    # the step as a serving loop runs it: write the new tokens, then attend over them
    sp = small("full_100k", batch=3, n_rows=4, kv_format=fmt, page_size=64,
               seq_len=("uniform", 200, 1500), dmax=2000, name="append_decode")
    case = synth.make_case(sp, seed=31)
    k_new, v_new = _new_rows(sp.batch, sp.n_rows, sp.num_kv_heads, sp.head_dim, seed=32)
    kc, vc, ks, vs, flags, _ = _append_both(case, k_new, v_new)
    assert flags == 0
    dev_case = dataclasses.replace(case.to("cuda"), k_cache=kc, v_cache=vc, k_scale=ks,
                                   v_scale=vs)
    out, lse, info, fl = run_hip(dev_case)
    assert fl == 0
    ok, ov, oks, ovs = _oracle_append(case, k_new, v_new)
    cpu_case = dataclasses.replace(case, k_cache=_from_codes(ok), v_cache=_from_codes(ov),
                                   k_scale=None if oks is None else torch.from_numpy(oks),
                                   v_scale=None if ovs is None else torch.from_numpy(ovs))
    ref_out, ref_lse, _ = oracle_of(cpu_case)
    compare(out, lse, ref_out, ref_lse, "append+decode %s" % fmt)


def test_append_skips_bad_rows():
    S, n = 16, 2
    sp = small("full_100k", batch=3, n_rows=n, kv_format=synth.KV_FP8, page_size=S,
               seq_len=("uniform", 40, 60), dmax=100, name="append_bad")
    case = synth.make_case(sp, seed=41)
    k_new, v_new = _new_rows(3, n, sp.num_kv_heads, sp.head_dim, seed=42)
    lens = case.seq_lens.clone()
    lens[1] = 1                                          # shorter than its 2 new tokens
    table = case.page_table.clone()
    L2 = int(lens[2])
    bad_page = (L2 - 1) // S
    table[2, bad_page] = 10 ** 6                         # the last token's page: outside
    say("append_bad lens=%s bad page %d of sequence 2" % (lens.tolist(), bad_page))
    kc, vc, ks, vs, flags, _ = _append_both(dataclasses.replace(case, page_table=table),
                                            k_new, v_new, seq_lens=lens)
    assert flags == (binding.RATTN_FLAG_SEQ_LEN_CLAMPED | binding.RATTN_FLAG_PAGE_CLAMPED)
    # expected: sequence 0 written in full, sequence 1 not at all, sequence 2 only the
    # tokens whose page id is valid
    want = [_as_codes(case.k_cache).copy(), _as_codes(case.v_cache).copy()]
    want_s = [case.k_scale.numpy().copy(), case.v_scale.numpy().copy()]
    for b in (0, 2):
        L = int(lens[b])
        for r in range(n):
            t = L - n + r
            if b == 2 and t // S == bad_page:
                continue
            page = int(case.page_table[b, t // S])
            for i, src in enumerate((k_new, v_new)):
                codes, sc = oracle.quantise_rows_e4m3(_as_codes(src[b, r]))
                want[i][page, :, t % S, :] = codes
                want_s[i][page, :, t % S] = sc
    _same_bits(_as_codes(kc), want[0], "K cache")
    _same_bits(_as_codes(vc), want[1], "V cache")
    _same_bits(ks, want_s[0], "K scales")
    _same_bits(vs, want_s[1], "V scales")
