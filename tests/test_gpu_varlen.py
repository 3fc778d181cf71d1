"""A different number of query rows per sequence (rattn_decode_varlen) on the GPU,
against the oracle's per-sequence definition.

Same floating-point bar as the fixed-row parity tests. The output buffers are filled
with NaN first: rows past the last sequence must stay NaN (bit for bit), and every
written row must match the oracle.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from decode_attention_verify_amd import binding, synth
from tests.parity import compare, say

pytestmark = pytest.mark.gpu


def small(base, **kw):
    return dataclasses.replace(synth.spec(base), **kw)


def run_varlen(case, q, cu, num_splits=0, extra_rows=3):
    """Packed rows on the GPU -> (out, lse, flags); out/lse hold extra rows past the last
    sequence, NaN-filled, which must stay untouched."""
    sp = case.spec
    dev = case.to("cuda")                     # no copy when the case is already there
    T = q.shape[0] + extra_rows
    qd = torch.zeros((T, sp.num_q_heads, sp.head_dim), dtype=torch.bfloat16, device="cuda")
    qd[:q.shape[0]] = q.to("cuda")
    out = torch.full((T, sp.num_q_heads, sp.head_dim), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((T, sp.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    prob = binding.problem_from_case(case, num_splits)
    with binding.Plan(prob) as plan:
        info = plan.info.as_dict()
        plan.decode_varlen(qd, dev.k_cache, dev.v_cache, dev.k_scale, dev.v_scale,
                           dev.page_table, dev.seq_lens, cu.to("cuda"), dev.bias, out, lse)
        torch.cuda.synchronize()
        flags = plan.debug_flags()
    say("  plan", info, "flags", flags)
    return out, lse, flags, q.shape[0]


def oracle_varlen(case, q, cu, batches=None, kv_heads=None):
    view = torch.uint16 if case.k_cache.dtype == torch.bfloat16 else torch.uint8
    sp = case.spec
    return oracle.relative_attention_varlen(
        q.view(torch.uint16).numpy(), cu.numpy(), case.k_cache.view(view).numpy(),
        case.v_cache.view(view).numpy(), case.page_table.numpy(), case.seq_lens.numpy(),
        case.bias.numpy(), window=sp.window, dmax=sp.dmax, softmax_scale=case.softmax_scale,
        k_scale=None if case.k_scale is None else case.k_scale.numpy(),
        v_scale=None if case.v_scale is None else case.v_scale.numpy(),
        batches=batches, kv_heads=kv_heads)


def check_varlen(sp, rows, seed, num_splits=0, gen_device="cpu", batches=None,
                 kv_heads=None):
    say("varlen %s rows=%s seed=%d splits=%d W=%d kv=%s" % (sp.name, rows, seed, num_splits,
                                                           sp.window, sp.kv_format))
    case = synth.make_case(sp, seed=seed, device=gen_device)
    cpu = case.to("cpu")
    q, cu = synth.varlen_rows(cpu, rows)
    out, lse, flags, T = run_varlen(case, q, cu, num_splits)
    assert flags == 0, "device flags %d on valid input" % flags
    assert bool(torch.isnan(out[T:].float()).all()), "rows past the last sequence written"
    assert bool(torch.isnan(lse[T:]).all()), "lse rows past the last sequence written"
    del case
    ref, ref_lse = oracle_varlen(cpu, q, cu, batches, kv_heads)
    if T:
        compare(out[:T], lse[:T], ref, ref_lse, "varlen %s" % sp.name)


@pytest.mark.parametrize("W", [0, 1024])
@pytest.mark.parametrize("seed", [0, 1])
def test_mixed_rows(W, seed):
    sp = small("window_b16", batch=9, n_rows=8, window=W, dmax=1500,
               seq_len=("uniform", 8, 1400), name="varlen")
    rows = synth.draw_rows_per_seq(9, 8, seed=seed)
    check_varlen(sp, rows, seed=seed)


@pytest.mark.parametrize("rows", [[1, 8, 0, 3], [0, 0, 5, 0], [8, 8, 8, 8], [2, 0, 0, 7]])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_rows_and_splits(rows, splits):
    sp = small("full_100k", batch=4, n_rows=8, seq_len=("uniform", 8, 2000), dmax=2500,
               name="varlen_splits")
    check_varlen(sp, rows, seed=sum(rows) + splits, num_splits=splits)


@pytest.mark.parametrize("k", [2, 3])
@pytest.mark.parametrize("rows", [[1, 2, 0, 2, 1], [0, 0, 2, 0, 0]])
def test_rows_of_merged_pieces(rows, k):
    # up to 2 rows of 6 heads: single-wave pieces; 2 or 3 per unit run as one work-group
    # that merges them, over sequences without rows and pieces without keys
    sp = small("full_100k", batch=5, n_rows=2, seq_len=("uniform", 2, 150), dmax=400,
               name="varlen_merge%d" % k)
    check_varlen(sp, rows, seed=sum(rows) + 30 + k, num_splits=k)


def test_no_rows_at_all():
    sp = small("full_100k", batch=3, n_rows=4, seq_len=("uniform", 4, 300), dmax=400,
               name="varlen_empty")
    check_varlen(sp, [0, 0, 0], seed=3)


@pytest.mark.parametrize("fmt", [synth.KV_BF16, synth.KV_FP8])
def test_mtp_rows_gqa4_window512(fmt):
    # the previous generation's sliding layers: 64 query / 16 KV heads, W = 512, and up to
    # 9 tokens per step from its MTP heads
    sp = small("v1_window_verify", batch=12, kv_format=fmt, page_size=64 if fmt == synth.KV_FP8
               else 16, seq_len=("uniform", 9, 3000), name="varlen_mtp")
    rows = synth.draw_rows_per_seq(12, 9, seed=7, allow_zero=False)
    check_varlen(sp, rows, seed=7)


def test_bad_row_ranges_are_flagged():
    sp = small("full_100k", batch=4, n_rows=4, seq_len=("uniform", 4, 500), dmax=600,
               name="varlen_bad")
    case = synth.make_case(sp, seed=9).to("cpu")
    q, cu = synth.varlen_rows(case, [2, 3, 1, 4])
    bad = cu.clone()
    bad[2] = bad[1] + 5                       # sequence 1 claims 5 rows (> n = 4)
    out, lse, flags, T = run_varlen(case, q, bad)
    assert flags & binding.RATTN_FLAG_ROWS_INVALID
    # sequences 0 and 3 are still right; sequence 1 wrote nothing
    ref, ref_lse = oracle_varlen(case, q, cu, batches=[0, 3])
    for b in (0, 3):
        s = slice(int(cu[b]), int(cu[b + 1]))
        compare(out[s], lse[s], ref[s], ref_lse[s], "valid sequence %d" % b)
    # rows 2..5 belonged to sequences 1 and 2, whose ranges are invalid
    assert int(cu[1]) == 2 and int(cu[3]) == 6
    assert bool(torch.isnan(lse[2:6].cpu()).all()) and bool(torch.isnan(out[2:6].float()).all())


@pytest.mark.parametrize("splits", [0, 5])
def test_rows_three_row_tiles(splits):
    # 1..8 rows of 6-head groups under a long planning bound: one wave of three row
    # tiles per piece, rows past a sequence's own count left out
    sp = small("full_100k", batch=9, n_rows=8, seq_len=("uniform", 8, 2500), dmax=3000,
               max_seq_len=9000, name="varlen_rows3")
    rows = synth.draw_rows_per_seq(9, 8, seed=21 + splits)
    check_varlen(sp, rows, seed=21 + splits, num_splits=splits)


@pytest.mark.parametrize("fmt", [synth.KV_BF16, synth.KV_FP8])
def test_mtp_rows_gqa8_full(fmt):
    # the previous generation's full layers (64q/8kv) with 1..9 tokens per sequence: up
    # to 72 packed rows, 8-wave work-groups
    sp = small("v1_full_mtp9", batch=7, kv_format=fmt, page_size=64 if fmt == synth.KV_FP8
               else 16, seq_len=("uniform", 9, 2500), dmax=3000, name="varlen_mtp9")
    rows = synth.draw_rows_per_seq(7, 9, seed=8)
    check_varlen(sp, rows, seed=8)


@pytest.mark.parametrize("fmt", [synth.KV_BF16, synth.KV_FP8])
def test_varlen_mtp9_full_size_sampled(fmt):
    sp = small("v1_full_mtp9_varlen", kv_format=fmt, page_size=64 if fmt == synth.KV_FP8
               else 16, name="v1_full_mtp9_varlen_" + fmt)
    rows = synth.draw_rows_per_seq(sp.batch, sp.n_rows, seed=sp.rows_seed, allow_zero=False)
    check_varlen(sp, rows, seed=0, gen_device="cuda", batches=[0, 3], kv_heads=[1, 6])


def test_varlen_verify_full_size_sampled():
    # the verify workload's shapes (16 sequences of 32K-256K keys) with 1..8 rows each
    sp = synth.spec("verify_b16")
    rows = synth.draw_rows_per_seq(16, 8, seed=11, allow_zero=False)
    check_varlen(sp, rows, seed=0, gen_device="cuda", batches=[2, 9], kv_heads=None)
