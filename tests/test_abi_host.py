"""The C-ABI library on the host: it loads, exports what include/rattn.h declares,
rejects invalid problems before any HIP call, and plans sensibly (no GPU needed)."""

import ctypes
import os
import re

import pytest

from decode_attention_verify_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rattn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rattn_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = binding.load()
    names = declared_functions()
    assert {"rattn_plan", "rattn_decode", "rattn_free"} <= set(names)
    for name in names:
        assert hasattr(lib, name), "librattn.so does not export %s" % name
    assert lib.rattn_abi_version() == binding.ABI_VERSION


def headline(**kw):
    base = dict(batch=1, num_q_heads=48, num_kv_heads=8, n_query_rows=1, page_size=16,
                num_pages=6251, max_pages_per_seq=6250, max_seq_len=100000, window=0,
                dmax=131071, softmax_scale=128 ** -0.5)
    base.update(kw)
    return binding.make_problem(**base)


INVALID = [
    dict(batch=0), dict(num_q_heads=0), dict(num_kv_heads=0), dict(num_q_heads=47),
    dict(n_query_rows=0), dict(page_size=0), dict(num_pages=0), dict(max_pages_per_seq=0),
    dict(max_seq_len=0), dict(max_seq_len=100001), dict(window=-1), dict(dmax=-1),
    dict(softmax_scale=float("inf")), dict(softmax_scale=float("nan")), dict(kv_dtype=2),
    # the scale must be a positive normal float (the kernels divide the bias by it)
    dict(softmax_scale=0.0), dict(softmax_scale=-0.08), dict(softmax_scale=1e-40),
    dict(num_splits=-1),
]
UNSUPPORTED = [
    dict(head_dim=64), dict(page_size=24, max_pages_per_seq=6250),
    # more than 128 packed rows go to the prefill kernel, built for G = 4, 6, 8 over a
    # bf16 cache without forced splits
    dict(n_query_rows=100, num_q_heads=24), dict(n_query_rows=100, num_splits=4),
    # a split grid of 2^31 work-items or more (a work-group of up to 8 waves per unit)
    dict(batch=1 << 19, max_seq_len=1, max_pages_per_seq=1),
    # the call's tiles are counted in 32-bit integers: 2^31 tiles or more are refused
    dict(batch=256, num_kv_heads=8, num_q_heads=48, max_seq_len=1 << 25,
         max_pages_per_seq=1 << 21, num_pages=1 << 21),
    dict(page_size=8, max_pages_per_seq=12500), dict(num_splits=4097),
    # 128 query heads per KV head: a tile's bias slice (128 x 32 distances) exceeds what
    # a work-group stages (64 per KV head fit an 8-wave group)
    dict(num_q_heads=1024, num_kv_heads=8),
]


@pytest.mark.parametrize("bad", INVALID)
def test_invalid_problems_rejected(bad):
    prob = headline(**bad)
    with pytest.raises(binding.RattnError) as e:
        binding.rattn_plan_describe(prob, 256)
    assert e.value.status == binding.RATTN_E_INVALID
    # rattn_plan validates before touching HIP, so this is safe without a GPU
    with pytest.raises(binding.RattnError) as e:
        binding.rattn_plan(prob)
    assert e.value.status == binding.RATTN_E_INVALID


@pytest.mark.parametrize("bad", UNSUPPORTED)
def test_unsupported_problems_rejected(bad):
    with pytest.raises(binding.RattnError) as e:
        binding.rattn_plan_describe(headline(**bad), 256)
    assert e.value.status == binding.RATTN_E_UNSUPPORTED


def test_null_arguments():
    lib = binding.load()
    assert lib.rattn_plan(None, None) == binding.RATTN_E_INVALID
    assert lib.rattn_plan_describe(None, 256, None) == binding.RATTN_E_INVALID
    assert lib.rattn_decode(*([None] * 12)) == binding.RATTN_E_INVALID
    assert lib.rattn_free(None) == binding.RATTN_OK
    assert lib.rattn_plan_get_info(None, None) == binding.RATTN_E_INVALID


def test_planner_headline_fills_the_chip():
    info = binding.rattn_plan_describe(headline(), 256)
    assert info.row_tiles == 1                 # 6 packed rows: one wave per piece
    assert info.grid_y == 1 and info.grid_z == 1
    # one round of resident work-groups (4 per CU on gfx950), three quarters full
    assert info.blocks_per_cu == 4
    assert info.pieces_per_group == 1
    assert info.grid_x == 256 * 4 * 3 // 4, info.grid_x
    units = 8
    assert info.grid_x * info.keys_per_split >= units * 100000
    assert info.keys_per_split % info.tile_keys == 0
    assert info.combine_blocks == 48 * 8   # 8 work-groups per output row


def test_planner_one_tile_pieces_when_units_are_few():
    # 2048 keys on one 6q/1kv unit: 65 tiles, each its own piece (the round of 768 pieces
    # is far from full); 8 window units of 1024 + 31 keys: 33 one-tile pieces each
    tiny = headline(num_q_heads=6, num_kv_heads=1, max_seq_len=2048, max_pages_per_seq=128,
                    dmax=2047)
    info = binding.rattn_plan_describe(tiny, 256)
    assert info.num_splits == 65 and info.grid_x == 65 and info.combine_blocks > 0
    window = headline(window=1024, max_seq_len=32768, max_pages_per_seq=2048)
    info = binding.rattn_plan_describe(window, 256)
    assert info.num_splits == 33 and info.grid_x == 8 * 33
    # where the round binds, the pieces stay longer: 16 window sequences, 6 pieces each
    info = binding.rattn_plan_describe(
        headline(batch=16, window=1024, max_seq_len=32768, max_pages_per_seq=2048), 256)
    assert info.num_splits == 6 and info.keys_per_split >= 4 * info.tile_keys


def test_planner_merges_three_pieces_in_one_group():
    # 64q/16kv window layer at batch 16: 256 units of 4 packed rows, three single-wave
    # pieces each, which one 3-wave work-group per unit attends and merges
    p = headline(batch=16, num_q_heads=64, num_kv_heads=16, window=512, dmax=512,
                 max_seq_len=32768, max_pages_per_seq=2048)
    info = binding.rattn_plan_describe(p, 256)
    assert info.num_splits == 3 and info.pieces_per_group == 3
    assert info.grid_x == 16 * 16 and info.combine_blocks == 0
    # 48q/8kv window layer at batch 64: 512 units, two merged pieces each (two 2-wave
    # work-groups per CU)
    p = headline(batch=64, window=1024, max_seq_len=32768, max_pages_per_seq=2048)
    info = binding.rattn_plan_describe(p, 256)
    assert info.num_splits == 2 and info.pieces_per_group == 2
    assert info.grid_x == 512 and info.combine_blocks == 0
    # twice the CUs' units or more: whole units, one wave each
    assert binding.rattn_plan_describe(p, 255).pieces_per_group == 1
    # a forced split in two or three pieces, whatever the shape, for single-wave bf16
    for k in (2, 3):
        for kw in (dict(), dict(batch=3), dict(n_query_rows=2)):
            info = binding.rattn_plan_describe(headline(num_splits=k, **kw), 256)
            assert info.pieces_per_group == k and info.combine_blocks == 0
            assert info.grid_x == headline(**kw).batch * 8
    # not for multi-wave pieces or an E4M3 cache
    for kw in (dict(n_query_rows=3), dict(kv_dtype=binding.RATTN_KV_FP8_E4M3)):
        info = binding.rattn_plan_describe(headline(num_splits=3, **kw), 256)
        assert info.pieces_per_group == 1 and info.combine_blocks > 0


def test_planner_covers_every_key():
    for kw in (dict(), dict(window=1024, max_seq_len=32768, max_pages_per_seq=2048),
               dict(batch=64, window=1024, max_seq_len=32768, max_pages_per_seq=2048),
               dict(batch=16, n_query_rows=8, max_seq_len=262144, max_pages_per_seq=16384,
                    dmax=262143),
               dict(num_splits=7), dict(num_splits=4096), dict(max_seq_len=1,
                                                                max_pages_per_seq=1)):
        p = headline(**kw)
        units = p.batch * p.num_kv_heads
        span = (min(p.max_seq_len, p.window + p.n_query_rows - 1) if p.window
                else p.max_seq_len) + 31
        tiles = -(-span // 32)
        for cus in (1, 80, 256, 304):
            info = binding.rattn_plan_describe(p, cus)
            ppg = info.pieces_per_group
            assert ppg in (1, 2, 3)
            pieces = info.grid_x * ppg
            assert pieces * info.keys_per_split >= units * tiles * 32
            if p.num_splits:
                assert pieces == min(p.num_splits * units, 1 << 16)
            else:
                assert pieces <= max(units, units * tiles)
            assert 1 <= info.grid_x <= 1 << 16
            rows = 6 * p.n_query_rows
            one_wave = 16 < rows <= 48 and p.window == 0 and p.max_seq_len >= 8192
            assert info.tiles_per_wave == (-(-rows // 16) if one_wave else 1)
            assert info.row_tiles == (1 if rows <= 16 or one_wave else 2 if rows <= 32 else
                                      4 if rows <= 64 else 8)
            if p.num_splits:
                assert ppg == (p.num_splits if p.num_splits in (2, 3) and rows <= 16 else 1)
            assert ppg in (1, 2, 3) and (ppg == 1 or ppg == info.num_splits)
            if ppg > 1:
                # one work-group per unit merges its pieces
                assert info.combine_blocks == 0 and info.grid_x == units
                assert rows <= 16 and units <= (cus if ppg == 3 else 2 * cus) or p.num_splits
            elif info.combine_blocks == 0:
                # nothing to merge: one work-group per (sequence, KV head) unit, or one in all
                assert info.grid_x in (1, units)
            else:
                assert info.workspace_bytes >= info.grid_x * rows * 129 * 4


def test_combine_shape_follows_the_pieces():
    # per-unit splits of up to 16 pieces merge whole rows, 4 per work-group; more, 8
    # work-groups per output row (16 dims each); 256 or more over 48 rows, 4 (32 dims)
    for k in (4, 7, 16, 17, 64, 255, 256, 4096):
        p = headline(num_splits=k)
        info = binding.rattn_plan_describe(p, 256)
        rows = p.batch * p.n_query_rows * p.num_q_heads
        want = -(-rows // 4) if k <= 16 else rows * 8 if k < 256 else rows * 4
        assert info.combine_blocks == want, (k, info.combine_blocks)
        assert info.pieces_per_group == 1
    # hundreds of pieces over few rows (one rank's share under 8-way tensor parallelism):
    # 16-dim slices
    tp8 = binding.rattn_plan_describe(headline(num_q_heads=6, num_kv_heads=1, num_splits=768), 256)
    assert tp8.num_splits == 768 and tp8.combine_blocks == 6 * 8
    window = binding.rattn_plan_describe(
        headline(batch=16, window=1024, max_seq_len=32768, max_pages_per_seq=2048), 256)
    assert 1 < window.num_splits <= 16 and window.combine_blocks == -(-16 * 48 // 4)
    # even shares of a full-context batch: whole rows, 4 per work-group
    verify = binding.rattn_plan_describe(
        headline(batch=16, n_query_rows=8, max_seq_len=262144, max_pages_per_seq=16384,
                 dmax=262143), 256)
    assert verify.combine_blocks == 16 * 8 * 48 // 4


@pytest.mark.parametrize("hq,n,tokens", [(48, 22, 64), (48, 2048, 64), (32, 33, 64),
                                         (64, 17, 32), (64, 1000, 32)])
def test_planner_prefill(hq, n, tokens):
    # more than 128 packed rows: one 8-wave prefill work-group per (sequence, KV head,
    # block of query tokens: 4 blocks of 16 for 6- and 4-head groups, 2 for 8-head
    # groups), a grid rounded up to a multiple of 8 (one share per XCD), no combine
    p = headline(batch=3, num_q_heads=hq, n_query_rows=n)
    info = binding.rattn_plan_describe(p, 256)
    assert info.kernel == binding.RATTN_KERNEL_PREFILL
    blocks = 3 * 8 * -(-n // tokens)
    assert info.grid_x % 8 == 0 and blocks <= info.grid_x < blocks + 8
    assert info.combine_blocks == 0 and info.row_tiles == 8
    assert binding.rattn_plan_describe(headline(), 256).kernel == binding.RATTN_KERNEL_SPLIT_KV
    # the same over an E4M3 cache
    p8 = headline(batch=3, num_q_heads=hq, n_query_rows=n, kv_dtype=binding.RATTN_KV_FP8_E4M3)
    info8 = binding.rattn_plan_describe(p8, 256)
    assert info8.kernel == binding.RATTN_KERNEL_PREFILL and info8.grid_x == info.grid_x


def test_read_probe_rejects_bad_arguments():
    lib = binding.load()
    vp = ctypes.c_void_p
    one = vp(16)                               # never dereferenced: rejected on the host
    for args in ((None, 4, 4096, None, 8, one, None), (one, 0, 4096, None, 8, one, None),
                 (one, 4, 1000, None, 8, one, None), (one, 4, 4096, None, 0, one, None),
                 (one, 4, 4096, None, 8, None, None)):
        assert lib.rattn_read_probe(*args) == binding.RATTN_E_INVALID


@pytest.mark.parametrize("hq,n", [(64, 9), (48, 11), (48, 21), (32, 32), (64, 16)])
@pytest.mark.parametrize("kv", [binding.RATTN_KV_BF16, binding.RATTN_KV_FP8_E4M3])
def test_planner_65_to_128_rows(hq, n, kv):
    # 65 to 128 packed rows (the 9-token step on 8-head groups: 72 rows) stay on the
    # split kernel: over a bf16 cache and long spans four waves of two row tiles each,
    # else one 16-row tile per wave in 8-wave work-groups (an E4M3 cache, a short span);
    # a full-context batch is shared evenly and merged by the combine
    G = hq // 8
    assert 64 < G * n <= 128
    want = (4, 2) if kv == binding.RATTN_KV_BF16 else (8, 1)
    p = headline(batch=4, num_q_heads=hq, n_query_rows=n, max_seq_len=262144,
                 max_pages_per_seq=16384, num_pages=65536, dmax=262143, kv_dtype=kv)
    info = binding.rattn_plan_describe(p, 256)
    assert info.kernel == binding.RATTN_KERNEL_SPLIT_KV
    assert (info.row_tiles, info.tiles_per_wave) == want
    assert info.pieces_per_group == 1 and info.combine_blocks == -(-4 * n * hq // 4)
    assert info.workspace_bytes >= (info.grid_x + 32) * G * n * 129 * 4
    # batch 1: the unit's keys cut into pieces of equal length
    one = binding.rattn_plan_describe(headline(num_q_heads=hq, n_query_rows=n, kv_dtype=kv), 256)
    assert (one.row_tiles, one.tiles_per_wave) == want
    assert one.num_splits > 1 and one.grid_x == 8 * one.num_splits
    # a window of 1,024 keys: one row tile per wave
    short = binding.rattn_plan_describe(
        headline(num_q_heads=hq, n_query_rows=n, kv_dtype=kv, window=1024, max_seq_len=32768,
                 max_pages_per_seq=2048), 256)
    assert (short.row_tiles, short.tiles_per_wave) == (8, 1)


def test_planner_two_row_tiles_bias_share():
    # four waves of two row tiles load a tile's bias slice with 2 loads per lane: a
    # 16-head group's slice (16 x 36 entries at n = 5) goes to 8-wave groups instead
    for hq, n, want in ((128, 5, (8, 1)), (128, 8, (8, 1)), (96, 6, (4, 2)), (64, 16, (4, 2))):
        G = hq // 8
        assert 64 < G * n <= 128
        assert (G * (32 + n - 1) <= 512) == (want == (4, 2))
        p = headline(batch=4, num_q_heads=hq, n_query_rows=n, max_seq_len=262144,
                     max_pages_per_seq=16384, num_pages=65536, dmax=262143)
        info = binding.rattn_plan_describe(p, 256)
        assert info.kernel == binding.RATTN_KERNEL_SPLIT_KV
        assert (info.row_tiles, info.tiles_per_wave) == want, (hq, n)


def test_static_entry_checks_on_the_host():
    # rattn_decode_static validates the problem and its pointers before any HIP call
    lib = binding.load()
    vp = ctypes.c_void_p
    one = vp(16)                               # never dereferenced: rejected on the host
    # q, k_cache, v_cache, k_scale, v_scale, page_table, seq_lens, bias, out, lse, flags,
    # stream: a bf16 cache takes no scales
    ptrs = [one, one, one, None, None, one, one, one, one, one, None, None]
    assert len(ptrs) == len(lib.rattn_decode_static.argtypes) - 1
    bad = headline(num_kv_heads=7)
    assert lib.rattn_decode_static(ctypes.byref(bad), *ptrs) == binding.RATTN_E_INVALID
    prob = headline()
    for i in (0, 1, 2, 5, 6, 7, 8):            # q, k, v, table, lengths, bias, out
        args = list(ptrs)
        args[i] = None
        assert lib.rattn_decode_static(ctypes.byref(prob), *args) == binding.RATTN_E_INVALID
    args = list(ptrs)
    args[3] = one                              # a scale array for a bf16 cache
    assert lib.rattn_decode_static(ctypes.byref(prob), *args) == binding.RATTN_E_INVALID
    fp8 = headline(kv_dtype=binding.RATTN_KV_FP8_E4M3)
    assert lib.rattn_decode_static(ctypes.byref(fp8), *ptrs) == binding.RATTN_E_INVALID


def test_planner_one_wave_of_three_row_tiles():
    # 17 to 48 packed rows over a bf16 cache whose rows see 8,192 keys or more: one wave
    # per piece holding two or three 16-row tiles; shorter spans (window layers), an E4M3
    # cache and other row counts keep the multi-wave groups
    verify = dict(batch=16, n_query_rows=8, max_seq_len=262144, max_pages_per_seq=16384,
                  dmax=262143)
    info = binding.rattn_plan_describe(headline(**verify), 256)
    assert info.row_tiles == 1 and info.tiles_per_wave == 3
    info = binding.rattn_plan_describe(headline(n_query_rows=6), 256)      # 36 rows, 100K
    assert info.row_tiles == 1 and info.tiles_per_wave == 3
    for n in (3, 5):                                                        # 18, 30 rows
        info = binding.rattn_plan_describe(headline(**dict(verify, n_query_rows=n)), 256)
        assert info.row_tiles == 1 and info.tiles_per_wave == 2
    for kw in (dict(verify, window=1024, dmax=1031), dict(verify, max_seq_len=8191),
               dict(verify, kv_dtype=binding.RATTN_KV_FP8_E4M3), dict(verify, n_query_rows=9)):
        info = binding.rattn_plan_describe(headline(**kw), 256)
        assert info.tiles_per_wave == 1 and info.row_tiles in (2, 4, 8), kw
