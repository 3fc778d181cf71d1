"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Bar (floating point): max-abs(out) <= 2e-2, mean-abs(out) <= 2e-3, and
|lse - lse_ref| / max(|lse_ref|, 1) <= 1e-3, over every compared element. Inputs are
NaN-poisoned wherever the method must not read, so a stray read fails the check.
"""

import dataclasses

import pytest
import torch

from decode_attention_verify_amd import binding, synth
from tests.parity import check_case, compare, oracle_of, run_hip, say

pytestmark = pytest.mark.gpu


def small(base, **kw):
    return dataclasses.replace(synth.spec(base), **kw)


# ---------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_full_context(seed):
    check_case(synth.spec("tiny"), seed=seed)


@pytest.mark.parametrize("name", ["window_b1", "window_b16", "window_b64"])
def test_sliding_window(name):
    check_case(synth.spec(name), seed=0, gen_device="cuda")


def test_window_verify_b16():
    check_case(synth.spec("window_verify_b16"), seed=0, gen_device="cuda")


def test_full_context_100k():
    check_case(synth.spec("full_100k"), seed=0, gen_device="cuda")


def test_verify_b16_sampled():
    sp = synth.spec("verify_b16")
    # all KV heads of sequences 0 and 5, plus KV head 3 of every sequence
    check_case(sp, seed=0, gen_device="cuda", batches=[0, 5], kv_heads=None)
    check_case(sp, seed=0, gen_device="cuda", batches=None, kv_heads=[3])


def test_fp8_1m_sampled():
    check_case(synth.spec("fp8_1m"), seed=0, gen_device="cuda", kv_heads=[0, 7])


# ------------------------------------ the previous generation's layer shapes (64q heads)

def test_v1_full_decode():
    check_case(synth.spec("v1_full_decode"), seed=0, gen_device="cuda")


def test_v1_window_decode():
    check_case(synth.spec("v1_window_decode"), seed=0, gen_device="cuda")


def test_v1_full_verify_sampled():
    check_case(synth.spec("v1_full_verify"), seed=0, gen_device="cuda", batches=[1],
               kv_heads=None)
    check_case(synth.spec("v1_full_verify"), seed=0, gen_device="cuda", kv_heads=[5])


def test_v1_window_verify():
    check_case(synth.spec("v1_window_verify"), seed=0, gen_device="cuda")


# ------------------- 65 to 128 packed rows: 8-wave work-groups (the 9-token MTP step)

def test_v1_full_mtp9_sampled():
    # the previous generation's full layer (64q/8kv) during a 9-token step: 72 packed rows
    sp = synth.spec("v1_full_mtp9")
    check_case(sp, seed=0, gen_device="cuda", batches=[1], kv_heads=None)
    check_case(sp, seed=0, gen_device="cuda", kv_heads=[5])


def test_v1_full_mtp9_fp8_sampled():
    sp = small("v1_full_mtp9", kv_format=synth.KV_FP8, page_size=64, name="v1_full_mtp9_fp8")
    check_case(sp, seed=1, gen_device="cuda", kv_heads=[2])


@pytest.mark.parametrize("hq,hkv,n,W,splits,batch,fmt", [
    (64, 8, 9, 0, 0, 5, synth.KV_BF16),       # even shares over mixed lengths
    (64, 8, 9, 0, 0, 5, synth.KV_FP8),
    (64, 8, 9, 0, 0, 1, synth.KV_BF16),       # one unit per KV head, cut into pieces
    (48, 8, 11, 1024, 0, 3, synth.KV_BF16),   # 66 rows over a window
    (48, 8, 21, 0, 3, 2, synth.KV_BF16),      # 126 rows, 3 forced pieces per unit
    (64, 8, 16, 17, 0, 3, synth.KV_FP8),      # 128 rows, window 17
    (32, 8, 32, 0, 7, 2, synth.KV_BF16),      # 4-head groups, 128 rows, 7 pieces
    (512, 8, 1, 0, 0, 2, synth.KV_BF16),      # 64 heads per KV head: the bias slice
])
def test_eight_wave_groups(hq, hkv, n, W, splits, batch, fmt):
    sp = small("full_100k", batch=batch, n_rows=n, num_q_heads=hq, num_kv_heads=hkv,
               window=W, kv_format=fmt, page_size=64 if fmt == synth.KV_FP8 else 16,
               seq_len=("uniform", n, 2600), dmax=3000, name="waves8")
    _, _, info = check_case(sp, seed=hq + n + W + splits + batch, num_splits=splits)
    assert info["row_tiles"] == 8


# ------- 33 to 48 packed rows over long spans: one wave holding three 16-row tiles

@pytest.mark.parametrize("n,batch,splits,dmax,lens", [
    (8, 12, 0, 3000, ("uniform", 8, 2000)),     # even shares over mixed lengths
    (6, 1, 7, 4000, 3000),                      # 36 rows, 7 pieces per unit
    (7, 3, 0, 37, ("uniform", 7, 1500)),        # 42 rows, the Dmax clamp
    (8, 2, 200, 3000, ("uniform", 8, 2500)),    # pieces without keys
    (3, 12, 0, 3000, ("uniform", 3, 2000)),     # 18 rows: two tiles, even shares
    (5, 1, 9, 4000, 3000),                      # 30 rows: two tiles, 9 pieces per unit
    (4, 3, 0, 29, ("uniform", 4, 1500)),        # 24 rows, the Dmax clamp
])
def test_row_tiles_per_wave(n, batch, splits, dmax, lens):
    # the planning bound (max_seq_len = 9,000) picks the one-wave layout of two or three
    # row tiles; the sequences themselves stay short so that the oracle checks every row
    sp = small("full_100k", batch=batch, n_rows=n, seq_len=lens, dmax=dmax, max_seq_len=9000,
               name="rows_rt")
    _, _, info = check_case(sp, seed=n + batch + splits, num_splits=splits, poison=dmax > 37)
    assert info["row_tiles"] == 1 and info["tiles_per_wave"] == -(-6 * n // 16)


# ---------------- batched full-context layers through the even-share variants, full size

@pytest.mark.parametrize("name,kv_head", [
    ("verify_b16_fp8", 3),     # E4M3, 48 rows: 4-wave groups
    ("decode_b16_fp8", 6),     # E4M3, 6 rows: one wave
    ("verify3_b16_fp8", 1),    # E4M3, 18 rows: 2-wave groups
])
def test_batched_full_layers_e4m3_sampled(name, kv_head):
    check_case(synth.spec(name), seed=0, gen_device="cuda", kv_heads=[kv_head])


def test_three_rows_short_contexts():
    # 18 packed rows, planning bound 8,191 keys: 2-wave groups, even shares; every unit
    check_case(synth.spec("verify3_b16_8k"), seed=0, gen_device="cuda")


# ----- 65 to 128 packed rows over long spans: four waves, each holding two row tiles

@pytest.mark.parametrize("hq,n,batch,splits,dmax,lens", [
    (64, 9, 6, 0, 3000, ("uniform", 9, 2000)),   # 72 rows (the 9-token step), even shares
    (64, 9, 1, 5, 4000, 3000),                   # 5 pieces per unit
    (64, 16, 2, 0, 45, ("uniform", 16, 1500)),   # 128 rows, the Dmax clamp
    (48, 11, 2, 300, 3000, ("uniform", 11, 2500)),   # 66 rows, pieces without keys
    (32, 20, 3, 0, 3000, ("uniform", 20, 2000)),     # 4-head groups, 80 rows
])
def test_four_waves_of_two_row_tiles(hq, n, batch, splits, dmax, lens):
    # the planning bound (max_seq_len = 9,000) picks the four-wave layout; rows per wave
    # spread evenly over the wave's two tiles; short sequences, so that the oracle checks
    # every row
    sp = small("full_100k", batch=batch, n_rows=n, num_q_heads=hq, num_kv_heads=8,
               seq_len=lens, dmax=dmax, max_seq_len=9000, name="rows_4x2")
    _, _, info = check_case(sp, seed=hq + n + batch + splits, num_splits=splits,
                            poison=dmax > 45)
    assert info["row_tiles"] == 4 and info["tiles_per_wave"] == 2


@pytest.mark.parametrize("splits,L", [(63, 2000), (32, 2000), (21, 2000), (13, 2000),
                                      (9, 2000), (2, 20000)])
def test_four_waves_two_tiles_in_flight(splits, L):
    # the four-wave layout keeps two tiles in flight; 63 tiles in 63, 32, 21, 13 and 9
    # pieces give pieces of 1 to 7 tiles (each way its tile loop can end), and 20,000 keys
    # in two pieces give pieces that span two chunks of page ids
    sp = small("full_100k", batch=1, n_rows=9, num_q_heads=64, num_kv_heads=8, seq_len=L,
               dmax=max(L, 9000), max_seq_len=max(L, 9000), name="rows_4x2_tails")
    _, _, info = check_case(sp, seed=splits, num_splits=splits)
    assert info["row_tiles"] == 4 and info["tiles_per_wave"] == 2


@pytest.mark.parametrize("n,batch", [(5, 2), (8, 1)])
def test_sixteen_head_groups_long_span(n, batch):
    # 80 and 128 packed rows of 16-head groups over more than 8,192 keys: their bias slice
    # (16 x (31 + n) entries) exceeds the two-row-tile layout's share, so 8-wave groups run
    sp = small("full_100k", batch=batch, n_rows=n, num_q_heads=16, num_kv_heads=1,
               seq_len=("uniform", 8500, 9500), dmax=9000, max_seq_len=9500, name="g16_long")
    _, _, info = check_case(sp, seed=n)
    assert info["row_tiles"] == 8 and info["tiles_per_wave"] == 1


# ------------------------- one GPU's share of the headline layer under TP4 / TP8 (KV heads)

@pytest.mark.parametrize("name", ["tp4_100k", "tp8_100k"])
def test_tensor_parallel_shares(name):
    check_case(synth.spec(name), seed=0, gen_device="cuda")


# ---------------------------------------------------------------- sweeps at small sizes

@pytest.mark.parametrize("n", range(1, 9))
@pytest.mark.parametrize("window", [0, 1, 17, 1024])
def test_rows_and_windows(n, window):
    sp = small("window_b16", batch=3, n_rows=n, window=window, dmax=1500,
               seq_len=("uniform", n, 300), name="sweep")
    check_case(sp, seed=10 * n + window)


@pytest.mark.parametrize("L", [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 1000, 1023, 1024, 1025])
def test_page_boundaries(L):
    n = min(L, 3)
    sp = small("full_100k", batch=2, n_rows=n, seq_len=L, dmax=2000, bias_decay=0.0,
               name="boundary")
    check_case(sp, seed=L)


@pytest.mark.parametrize("splits", [1, 2, 7, 64, 4096])
def test_forced_splits(splits):
    sp = small("full_100k", batch=2, n_rows=2, seq_len=("uniform", 500, 3000), dmax=4000,
               name="splits")
    check_case(sp, seed=5, num_splits=splits)


@pytest.mark.parametrize("page_size", [16, 32, 64, 256])
@pytest.mark.parametrize("fmt", [synth.KV_BF16, synth.KV_FP8])
def test_page_sizes_and_formats(page_size, fmt):
    sp = small("full_100k", batch=3, n_rows=4, page_size=page_size, kv_format=fmt,
               seq_len=("uniform", 100, 2500), dmax=3000, name="pages")
    check_case(sp, seed=page_size)


@pytest.mark.parametrize("hq,hkv,n", [(64, 8, 8), (64, 16, 8), (48, 8, 9), (32, 8, 16),
                                      (8, 8, 8), (6, 1, 10)])
def test_gqa_ratios(hq, hkv, n):
    sp = small("full_100k", batch=2, n_rows=n, num_q_heads=hq, num_kv_heads=hkv,
               seq_len=("uniform", 200, 1500), dmax=2000, name="gqa")
    check_case(sp, seed=hq + hkv + n)


@pytest.mark.parametrize("n", [1, 3, 8])
def test_even_shares_across_units(n):
    # a full-context batch of mixed lengths is shared evenly among the work-groups, so
    # a work-group's tiles run across several (sequence, KV head) units and most units
    # are split between two work-groups at arbitrary tile boundaries
    sp = small("full_100k", batch=12, n_rows=n, seq_len=("uniform", n, 700), dmax=1000,
               name="even")
    check_case(sp, seed=20 + n)


def test_dmax_clamp_on_gpu():
    sp = small("full_100k", batch=2, n_rows=5, seq_len=("uniform", 300, 900), dmax=37,
               name="dmax")
    check_case(sp, seed=3, poison=False)


@pytest.mark.parametrize("dmax", [0, 1, 2, 3, 4, 37])
@pytest.mark.parametrize("n", [1, 2])
def test_dmax_clamp_single_wave(dmax, n):
    # 6 n <= 16 rows: one wave per piece, which reads its bias as four adjacent table
    # entries per 16-byte load; tables of fewer than four entries per head, and tiles
    # whose distances pass Dmax or run below zero, take the entries one by one
    sp = small("full_100k", batch=3, n_rows=n, seq_len=("uniform", 300, 900), dmax=dmax,
               name="dmax1")
    check_case(sp, seed=40 + dmax, poison=False)


@pytest.mark.parametrize("dmax", [2, 45])
def test_dmax_clamp_fp8_single_wave(dmax):
    sp = small("fp8_1m", batch=2, seq_len=("uniform", 200, 1500), dmax=dmax, name="dmax_fp8")
    check_case(sp, seed=50 + dmax, poison=False)


@pytest.mark.parametrize("L", [100001, 100002, 100003])
def test_full_context_unaligned_lengths(L):
    # every length modulo 4: the bias entries of a 16-byte load start at any 4-byte
    # boundary of the table
    check_case(small("full_100k", seq_len=L), seed=0, gen_device="cuda", kv_heads=[2, 5])


@pytest.mark.parametrize("k", [2, 3])
@pytest.mark.parametrize("n,seq_len", [(1, ("uniform", 1, 300)), (2, ("uniform", 2, 2500)),
                                       (1, 4099)])
def test_pieces_merged_in_one_group(k, n, seq_len):
    # a unit split in 2 or 3 single-wave pieces runs as one work-group of as many waves,
    # which merges them (no combine launch); short sequences leave pieces without keys
    sp = small("full_100k", batch=5, n_rows=n, seq_len=seq_len, dmax=5000, bias_decay=0.0,
               name="merge%d" % k)
    check_case(sp, seed=60 + 10 * k + n, num_splits=k)


@pytest.mark.parametrize("k", [2, 3])
def test_pieces_merged_window(k):
    sp = small("window_b16", batch=4, n_rows=1, name="merge%d_window" % k)
    check_case(sp, seed=63 + k, num_splits=k)


@pytest.mark.parametrize("splits,seq_len", [(300, 5000), (1000, 5000), (256, 20000)])
def test_many_pieces_few_rows(splits, seq_len):
    # hundreds of pieces over fewer than 32 rows: the combine's 16-dim slices of 256
    # stripes; at 5,000 keys (157 tiles) most pieces hold no key and are skipped
    sp = small("tiny", batch=2, n_rows=2, seq_len=seq_len, dmax=seq_len + 10,
               permute_pages=True, name="wide16")
    check_case(sp, seed=splits, num_splits=splits)


@pytest.mark.parametrize("W,n", [(1024, 8), (1, 1), (1, 8), (2, 3)])
def test_window_fp8(W, n):
    # windows of one or two keys: a row's output is one or two dequantised V rows, which
    # the P x V-scale products must carry to within the output's bf16 rounding
    sp = small("window_b16", batch=4, n_rows=n, window=W, kv_format=synth.KV_FP8,
               page_size=64, name="window_fp8")
    check_case(sp, seed=4 + W + n)


# ------------------------------------------------ one plan reused with different inputs

def _redrawn(case, seed):
    """The case's shapes, lengths, pages and NaN poison with new q, K, V and bias values
    (E4M3 codes redrawn among the finite ones)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    new = dataclasses.replace(case, seed=seed, q=case.q.clone(), k_cache=case.k_cache.clone(),
                              v_cache=case.v_cache.clone(), bias=case.bias.clone())
    new.q.copy_(torch.randn(case.q.shape, generator=g, device="cuda").to(torch.bfloat16))
    for c in (new.k_cache, new.v_cache):
        if c.dtype == torch.bfloat16:
            r = torch.randn(c.shape, generator=g, device="cuda").to(torch.bfloat16)
            c.copy_(torch.where(torch.isnan(c), c, r))
        else:
            r = torch.randint(0, 0x7F, c.shape, generator=g, device="cuda").to(torch.uint8)
            r |= (torch.randint(0, 2, c.shape, generator=g, device="cuda") * 0x80).to(torch.uint8)
            c.copy_(torch.where((c & 0x7F) == 0x7F, c, r))
    b = 0.5 * torch.randn(case.bias.shape, generator=g, device="cuda")
    new.bias.copy_(torch.where(torch.isfinite(case.bias), b, case.bias))
    return new


@pytest.mark.parametrize("base,kw,splits", [
    ("window_b16", dict(), 0),                                          # 6 pieces + combine
    ("window_b16", dict(batch=5, n_rows=2, seq_len=("uniform", 2, 400)), 8),   # empty pieces
    ("fp8_1m", dict(batch=3, n_rows=2, seq_len=("uniform", 50, 3000), dmax=3000), 5),
    ("tiny", dict(batch=2, seq_len=("uniform", 1, 700), dmax=800, permute_pages=True), 3),
    ("verify_b16", dict(batch=5, seq_len=("loguniform", 200, 9000)), 0),   # even shares
])
def test_plan_reused_with_alternating_inputs(base, kw, splits):
    # two input sets of the same shapes alternate through one plan, whose workspace
    # (partials, unit records) they share: every call must give its own inputs' output
    # bit for bit (a merge that read another call's partials would not); the first
    # output of each set is checked against the oracle
    sp = small(base, name="lastmerge", **kw)
    first = synth.make_case(sp, seed=31, device="cuda", poison=True)
    cases = [first, _redrawn(first, seed=32)]
    prob = binding.problem_from_case(cases[0], splits)
    shape = (sp.batch, sp.n_rows, sp.num_q_heads)
    with binding.Plan(prob) as plan:
        say("reused plan", plan.info.as_dict())
        refs = []
        for i in range(24):
            c = cases[i % 2]
            out = torch.empty(shape + (sp.head_dim,), dtype=torch.bfloat16, device="cuda")
            lse = torch.empty(shape, dtype=torch.float32, device="cuda")
            plan.decode(c.q, c.k_cache, c.v_cache, c.k_scale, c.v_scale, c.page_table,
                        c.seq_lens, c.bias, out, lse)
            if i < 2:
                refs.append((out, lse))
            else:
                ro, rl = refs[i % 2]
                assert torch.equal(out, ro) and torch.equal(lse, rl), "call %d" % i
        torch.cuda.synchronize()
        assert plan.debug_flags() == 0
    for (out, lse), c in zip(refs, cases):
        ref, ref_lse, _ = oracle_of(c.to("cpu"))
        compare(out, lse, ref, ref_lse, "reused plan, seed %d" % c.seed)


# ---------------------------------------------------------------- properties

def test_deterministic():
    sp = small("full_100k", batch=2, n_rows=8, seq_len=("uniform", 3000, 9000), name="det")
    case = synth.make_case(sp, seed=7).to("cuda")
    o1, l1, _, _ = run_hip(case)
    o2, l2, _, _ = run_hip(case)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "two runs differ"


def test_nonzero_stream():
    sp = small("full_100k", batch=2, n_rows=3, seq_len=2000, name="stream")
    case = synth.make_case(sp, seed=8).to("cuda")
    o1, l1, _, _ = run_hip(case)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2, l2, _, _ = run_hip(case, stream=s)
    s.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
