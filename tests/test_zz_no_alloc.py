"""rattn_decode_static (no allocation: partials in the library's static device array)
against rattn_decode (partials in the plan's workspace), through the C ABI on the GPU.

Several calls in a row share the one array, each with a smaller input than the one
before, so a call that depended on what an earlier one left in the array would show
here. The bar is the floating-point bar of the parity tests (max-abs 2e-2, mean-abs
2e-3, lse relative 1e-3); the two entry points launch the same kernels with the same
launch shape, so their outputs are also expected to be bitwise equal.
"""

import dataclasses

import numpy as np
import pytest
import torch

from decode_attention_verify_amd import binding, synth
from tests.parity import LSE_REL, MAX_ABS, MEAN_ABS, say

pytestmark = pytest.mark.gpu


def _run_both(sp, seed, num_splits=0):
    case = synth.make_case(sp, seed=seed, device="cuda", poison=True)
    prob = binding.problem_from_case(case, num_splits)
    shape = (sp.batch, sp.n_rows, sp.num_q_heads)
    outs = []
    for entry in ("plan", "static"):
        out = torch.full(shape + (sp.head_dim,), float("nan"), dtype=torch.bfloat16,
                         device="cuda")
        lse = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        flags = torch.zeros(1, dtype=torch.int32, device="cuda")
        if entry == "plan":
            with binding.Plan(prob) as plan:
                info = plan.info.as_dict()
                plan.decode(case.q, case.k_cache, case.v_cache, case.k_scale, case.v_scale,
                            case.page_table, case.seq_lens, case.bias, out, lse)
                torch.cuda.synchronize()
                assert plan.debug_flags() == 0
        else:
            binding.rattn_decode_static(prob, case.q, case.k_cache, case.v_cache, case.k_scale,
                                        case.v_scale, case.page_table, case.seq_lens,
                                        case.bias, out, lse, flags=flags)
            torch.cuda.synchronize()
            assert int(flags.item()) == 0, "device flags on valid input"
        outs.append((out, lse))
    say("  plan", info)
    return outs


def _check(sp, seed, num_splits=0):
    say("static vs plan: %s B=%d n=%d Hq=%d Hkv=%d W=%d kv=%s L=%s splits=%d" % (
        sp.name, sp.batch, sp.n_rows, sp.num_q_heads, sp.num_kv_heads, sp.window,
        sp.kv_format, sp.seq_len, num_splits))
    (o1, l1), (o2, l2) = _run_both(sp, seed, num_splits)
    a, b = o1.float().cpu().numpy(), o2.float().cpu().numpy()
    la, lb = l1.cpu().numpy().astype(np.float64), l2.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b)), "non-finite output"
    d = np.abs(a - b)
    rel = np.abs(la - lb) / np.maximum(np.abs(la), 1.0)
    say("  max_abs=%.3g mean_abs=%.3g lse_rel=%.3g bitwise_equal=%s" % (
        d.max(), d.mean(), rel.max(), bool(torch.equal(o1, o2) and torch.equal(l1, l2))))
    assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS and rel.max() <= LSE_REL


def test_static_entry_matches_plan_entry_on_shrinking_calls():
    # 1) the 100K-key decode: 96 pieces per unit and the combine
    _check(synth.spec("full_100k"), seed=0)
    # 2) a smaller verify-shaped batch: even shares across units
    _check(dataclasses.replace(synth.spec("verify_b16"), batch=6,
                               seq_len=("loguniform", 2000, 20000), name="static_verify"),
           seed=1)
    # 3) smaller still: E4M3 cache, 7 forced pieces per unit
    _check(dataclasses.replace(synth.spec("fp8_1m"), batch=2, n_rows=2,
                               seq_len=("uniform", 100, 3000), dmax=3000,
                               name="static_fp8"), seed=2, num_splits=7)
    # 4) the smallest: a window layer of 3 sequences, two pieces merged in one work-group
    _check(dataclasses.replace(synth.spec("window_b16"), batch=3, name="static_window"),
           seed=3, num_splits=2)


def test_static_entry_refuses_partials_beyond_the_array():
    # 4096 forced pieces for each of 16 x 8 units of 48 rows: about 1.6 GB of partials
    sp = dataclasses.replace(synth.spec("verify_b16"), seq_len=("uniform", 40, 60),
                             name="static_too_big")
    case = synth.make_case(sp, seed=4, device="cuda", poison=False)
    prob = binding.problem_from_case(case, 4096)
    out = torch.empty((sp.batch, sp.n_rows, sp.num_q_heads, sp.head_dim), dtype=torch.bfloat16,
                      device="cuda")
    with pytest.raises(binding.RattnError) as e:
        binding.rattn_decode_static(prob, case.q, case.k_cache, case.v_cache, case.k_scale,
                                    case.v_scale, case.page_table, case.seq_lens, case.bias,
                                    out)
    assert e.value.status == binding.RATTN_E_UNSUPPORTED
