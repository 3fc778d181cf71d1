"""Chunked prefill (many query rows per sequence) on the GPU against the oracle.

Same floating-point bar as the decode parity tests. Small shapes compare every row;
the page's prefill workload (8 chunks of 2048 tokens at 100K context) compares sampled
rows, each computed by the oracle as a one-row decode of the first L - (n - 1 - r) keys
(a row of a chunk attends exactly as the last row of that shorter sequence).
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from decode_attention_verify_amd import binding, synth
from tests.parity import check_case, compare, run_hip, say

pytestmark = pytest.mark.gpu


def small(base, **kw):
    return dataclasses.replace(synth.spec(base), **kw)


@pytest.mark.parametrize("n,lens,W", [(22, (22, 40), 0), (65, (65, 700), 0),
                                      (100, (100, 1500), 0), (257, (300, 2100), 0),
                                      (96, (96, 900), 1), (130, (200, 3000), 64),
                                      (128, (128, 2000), 1024)])
def test_prefill_rows_windows(n, lens, W):
    sp = small("full_100k", batch=2, n_rows=n, seq_len=("uniform",) + lens, window=W,
               dmax=3500, name="prefill")
    _, _, info = check_case(sp, seed=n + W)
    assert info["kernel"] == binding.RATTN_KERNEL_PREFILL


@pytest.mark.parametrize("hq,hkv", [(32, 8), (64, 16), (64, 8), (48, 8)])
@pytest.mark.parametrize("page_size", [16, 64, 256])
def test_prefill_groups_and_pages(hq, hkv, page_size):
    sp = small("full_100k", batch=2, n_rows=80, num_q_heads=hq, num_kv_heads=hkv,
               page_size=page_size, seq_len=("uniform", 80, 1200), dmax=1300,
               name="prefill_g")
    check_case(sp, seed=hq + hkv + page_size)


@pytest.mark.parametrize("hq,hkv,n,W,page_size", [
    (48, 8, 22, (0), 64), (48, 8, 100, 64, 16), (64, 8, 40, 0, 64), (32, 8, 66, 1024, 256),
    (48, 8, 257, 1, 64),
])
def test_prefill_fp8_cache(hq, hkv, n, W, page_size):
    # chunks over an E4M3 cache with fp32 per-token-per-head scales: the codes decoded
    # exactly to bf16, K scales on the logit columns, V scales on P
    sp = small("full_100k", batch=2, n_rows=n, num_q_heads=hq, num_kv_heads=hkv, window=W,
               kv_format=synth.KV_FP8, page_size=page_size, seq_len=("uniform", n, 2200),
               dmax=2500, name="prefill_fp8")
    _, _, info = check_case(sp, seed=n + hq + W)
    assert info["kernel"] == binding.RATTN_KERNEL_PREFILL


@pytest.mark.parametrize("W,dmax", [(0, 45), (64, 45), (0, 0), (1, 0), (1, 7), (2, 1)])
def test_prefill_dmax_clamp(W, dmax):
    # most distances past Dmax: every clamped entry of a bias slice (stored in reverse in
    # LDS) is the table's last column; Dmax = 0 gives every key one bias, and a window of
    # one key leaves each row its own key alone
    sp = small("full_100k", batch=2, n_rows=100, seq_len=("uniform", 100, 1500), window=W,
               dmax=dmax, name="prefill_dmax")
    _, _, info = check_case(sp, seed=45 + W + dmax)
    assert info["kernel"] == binding.RATTN_KERNEL_PREFILL


def test_prefill_whole_sequence_is_the_chunk():
    # the first chunk of a prompt: L = n, every row causal over the chunk alone
    sp = small("full_100k", batch=3, n_rows=200, seq_len=200, dmax=250, bias_decay=0.0,
               name="prefill_first")
    check_case(sp, seed=4)


@pytest.mark.parametrize("name", ["prefill_8x2k", "prefill_8x2k_fp8", "prefill_4x2k_g8",
                                  "prefill_4x2k_g4"])
def test_prefill_full_size_sampled(name):
    sp = synth.spec(name)
    say("prefill full size: %s B=%d n=%d L=%s kv=%s" % (sp.name, sp.batch, sp.n_rows,
                                                       sp.seq_len, sp.kv_format))
    case = synth.make_case(sp, seed=0, device="cuda")
    out, lse, info, flags = run_hip(case)
    assert flags == 0 and info["kernel"] == binding.RATTN_KERNEL_PREFILL
    cpu = case.to("cpu")
    del case
    view = torch.uint16 if cpu.k_cache.dtype == torch.bfloat16 else torch.uint8
    kc, vc = cpu.k_cache.view(view).numpy(), cpu.v_cache.view(view).numpy()
    ks = None if cpu.k_scale is None else cpu.k_scale.numpy()
    vs = None if cpu.v_scale is None else cpu.v_scale.numpy()
    G = sp.num_q_heads // sp.num_kv_heads
    rng = np.random.default_rng(0)
    picks = [(b, r, g) for b, r, g in zip(rng.integers(0, sp.batch, 12),
                                          rng.integers(0, sp.n_rows, 12),
                                          rng.integers(0, sp.num_kv_heads, 12))]
    B, H = sp.batch, sp.num_kv_heads
    picks += [(0, 0, 0), (B - 1, sp.n_rows - 1, H - 1), (min(3, B - 1), 1023, min(2, H - 1))]
    for b, r, g in picks:
        L = int(cpu.seq_lens[b])
        q1 = cpu.q[b:b + 1, r:r + 1].contiguous().view(torch.uint16).numpy()
        o1, l1 = oracle.relative_attention(
            q1, kc, vc, cpu.page_table[b:b + 1].numpy(),
            np.array([L - (sp.n_rows - 1 - r)]), cpu.bias.numpy(), n_query_rows=1,
            window=sp.window, dmax=sp.dmax, softmax_scale=cpu.softmax_scale,
            k_scale=ks, v_scale=vs, kv_heads=[int(g)])
        hs = slice(g * G, (g + 1) * G)
        compare(out[b, r, hs].unsqueeze(0), lse[b, r, hs].unsqueeze(0), o1[0, 0, hs][None],
                l1[0, 0, hs][None], "prefill b=%d r=%d g=%d" % (b, r, g))
