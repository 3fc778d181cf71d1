"""Seeded random problem shapes against the oracle: group sizes, KV heads, rows per
sequence (including chunks that take the prefill kernel), windows, Dmax below the
reachable distances, page sizes, both cache formats and forced split counts, drawn
together so that their combinations, not only each feature alone, meet the oracle.
Unused cache slots, pages and bias columns hold NaN (``poison``). The split-kernel
problems run again with a seeded number of rows per sequence (0 allowed) through
rattn_decode_varlen, and every other problem's shapes append n new tokens per sequence
(rattn_append_kv), compared bit for bit."""

import dataclasses
import math

import numpy as np
import pytest

from decode_attention_verify_amd import binding, synth

from tests.parity import check_case
from tests.test_gpu_append import _append_both, _as_codes, _new_rows, _oracle_append, _same_bits
from tests.test_gpu_varlen import check_varlen

kMaxRows = 128          # packed rows above which a call takes the prefill kernel


def random_cases(count=64, seed=7121):
    """``count`` valid problems: (spec fields, forced split count, input seed)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 6, 8]))
        if G * hkv > 64:
            continue
        prefill = G in (4, 6, 8) and rng.random() < 0.15
        n = int(rng.integers(kMaxRows // G + 1, 40)) if prefill else int(rng.integers(1, 17))
        if not prefill:
            n = min(n, kMaxRows // G)
        fmt = synth.KV_FP8 if rng.random() < 0.35 else synth.KV_BF16
        W = 0 if rng.random() < 0.5 else int(rng.integers(1, 3000))
        S = int(rng.choice([16, 32, 64, 128]))
        B = int(rng.integers(1, 6))
        # lengths past 8,192 keys reach the layouts of several row tiles per wave
        Lmax = int(rng.integers(8192, 12001)) if rng.random() < 0.4 else int(rng.integers(64, 8192))
        Lmax = max(Lmax, n)
        Lmin = n if rng.random() < 0.5 else max(n, Lmax // 2)
        dmax = int(rng.integers(0, 100)) if rng.random() < 0.3 else Lmax + int(rng.integers(0, 50))
        splits = 0 if (prefill or rng.random() < 0.7) else int(rng.integers(1, 65))
        keys = min(Lmax, W + n) if W else Lmax        # keys one row can see, at most
        if B * G * hkv * n * keys > 4e7:               # keep the oracle to seconds
            B = 1
        if B * G * hkv * n * keys > 4e7:
            continue
        fields = dict(batch=B, n_rows=n, num_q_heads=G * hkv, num_kv_heads=hkv, window=W,
                      dmax=dmax, page_size=S, kv_format=fmt,
                      seq_len=("uniform", Lmin, Lmax))
        out.append((fields, splits, int(rng.integers(0, 1 << 30))))
    return out


CASES = random_cases()


def spec_of(i):
    fields, splits, seed = CASES[i]
    return dataclasses.replace(synth.spec("full_100k"), name="random%d" % i, **fields), splits, seed


def test_random_cases_plan():
    # every drawn problem is valid and goes to the kernel its row count implies
    for i in range(len(CASES)):
        sp, splits, _ = spec_of(i)
        L = sp.seq_len_bound()
        prob = binding.make_problem(
            batch=sp.batch, num_q_heads=sp.num_q_heads, num_kv_heads=sp.num_kv_heads,
            n_query_rows=sp.n_rows, page_size=sp.page_size,
            num_pages=sp.batch * math.ceil(L / sp.page_size) + 1,
            max_pages_per_seq=math.ceil(L / sp.page_size), max_seq_len=L, window=sp.window,
            dmax=sp.dmax, softmax_scale=1 / math.sqrt(sp.head_dim),
            kv_dtype=binding.RATTN_KV_FP8_E4M3 if sp.kv_format == synth.KV_FP8
            else binding.RATTN_KV_BF16,
            num_splits=splits, head_dim=sp.head_dim)
        info = binding.rattn_plan_describe(prob, 256)
        rows = sp.n_rows * sp.num_q_heads // sp.num_kv_heads
        want = (binding.RATTN_KERNEL_PREFILL if rows > kMaxRows
                else binding.RATTN_KERNEL_SPLIT_KV)
        assert info.kernel == want, (i, rows, info.kernel)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(len(CASES)))
def test_random_shapes(i):
    sp, splits, seed = spec_of(i)
    check_case(sp, seed=seed, num_splits=splits)


def _split_kernel(i):
    fields = CASES[i][0]
    return fields["n_rows"] * fields["num_q_heads"] // fields["num_kv_heads"] <= kMaxRows


@pytest.mark.gpu
@pytest.mark.parametrize("i", [i for i in range(len(CASES)) if _split_kernel(i)])
def test_random_shapes_varlen(i):
    sp, splits, seed = spec_of(i)
    rows = synth.draw_rows_per_seq(sp.batch, sp.n_rows, seed=seed, allow_zero=True)
    check_varlen(sp, rows, seed, num_splits=splits)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(0, len(CASES), 2))
def test_random_shapes_append(i):
    sp, _, seed = spec_of(i)
    case = synth.make_case(sp, seed=seed)
    k_new, v_new = _new_rows(sp.batch, sp.n_rows, sp.num_kv_heads, sp.head_dim, seed=seed)
    kc, vc, ks, vs, flags, _ = _append_both(case, k_new, v_new)
    assert flags == 0
    ok, ov, oks, ovs = _oracle_append(case, k_new, v_new)
    _same_bits(_as_codes(kc), ok, "K cache")
    _same_bits(_as_codes(vc), ov, "V cache")
    if sp.kv_format == synth.KV_FP8:
        _same_bits(ks, oks, "K scales")
        _same_bits(vs, ovs, "V scales")
