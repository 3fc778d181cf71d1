"""Helpers for the GPU parity tests: run the HIP path through the C ABI, run the
oracle on the same inputs, compare element by element."""

import sys
import time

import numpy as np
import torch

import oracle
from decode_attention_verify_amd import binding, synth

# acceptance bar for floating point (the problem statement's tolerances)
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_REL = 1e-3


def say(*args):
    print("[parity]", *args, flush=True)
    sys.stdout.flush()


def run_hip(case, num_splits=0, stream=None):
    """case on the GPU -> (out bf16, lse fp32, plan info dict, debug flags)."""
    sp = case.spec
    prob = binding.problem_from_case(case, num_splits)
    out = torch.empty((sp.batch, sp.n_rows, sp.num_q_heads, sp.head_dim), dtype=torch.bfloat16,
                      device=case.q.device)
    lse = torch.empty((sp.batch, sp.n_rows, sp.num_q_heads), dtype=torch.float32,
                      device=case.q.device)
    with binding.Plan(prob) as plan:
        info = plan.info.as_dict()
        plan.decode(case.q, case.k_cache, case.v_cache, case.k_scale, case.v_scale,
                    case.page_table, case.seq_lens, case.bias, out, lse, stream=stream)
        torch.cuda.synchronize()
        flags = plan.debug_flags()
    return out, lse, info, flags


def oracle_of(case_cpu, batches=None, kv_heads=None):
    a = case_cpu
    view = torch.uint16 if a.k_cache.dtype == torch.bfloat16 else torch.uint8
    sp = a.spec
    t0 = time.time()
    out, lse = oracle.relative_attention(
        a.q.view(torch.uint16).numpy(), a.k_cache.view(view).numpy(),
        a.v_cache.view(view).numpy(), a.page_table.numpy(), a.seq_lens.numpy(),
        a.bias.numpy(), n_query_rows=sp.n_rows, window=sp.window, dmax=sp.dmax,
        softmax_scale=a.softmax_scale,
        k_scale=None if a.k_scale is None else a.k_scale.numpy(),
        v_scale=None if a.v_scale is None else a.v_scale.numpy(),
        batches=batches, kv_heads=kv_heads)
    return out, lse, time.time() - t0


def compare(out, lse, ref_out, ref_lse, what=""):
    """Element-wise check on the entries the oracle computed (non-NaN in ref)."""
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    sel = ~np.isnan(ref_lse)
    assert sel.any(), "nothing to compare"
    osel = np.broadcast_to(sel[..., None], ref_out.shape)
    d = np.abs(o[osel] - ref_out[osel])
    max_abs, mean_abs = float(d.max()), float(d.mean())
    rel = np.abs(l[sel] - ref_lse[sel]) / np.maximum(np.abs(ref_lse[sel]), 1.0)
    lse_rel = float(rel.max())
    say("%s max_abs=%.3g mean_abs=%.3g lse_rel=%.3g (n=%d rows)" % (what, max_abs, mean_abs,
                                                                    lse_rel, int(sel.sum())))
    assert np.all(np.isfinite(o[osel])) and np.all(np.isfinite(l[sel])), "non-finite output"
    assert max_abs <= MAX_ABS, "max-abs %g > %g" % (max_abs, MAX_ABS)
    assert mean_abs <= MEAN_ABS, "mean-abs %g > %g" % (mean_abs, MEAN_ABS)
    assert lse_rel <= LSE_REL, "lse rel %g > %g" % (lse_rel, LSE_REL)
    return max_abs, mean_abs, lse_rel


def check_case(sp, seed=0, num_splits=0, batches=None, kv_heads=None, gen_device="cpu",
               poison=True):
    say("case %s seed=%d splits=%d B=%d n=%d Hq=%d Hkv=%d W=%d S=%d kv=%s L=%s" % (
        sp.name, seed, num_splits, sp.batch, sp.n_rows, sp.num_q_heads, sp.num_kv_heads,
        sp.window, sp.page_size, sp.kv_format, sp.seq_len))
    case = synth.make_case(sp, seed=seed, device=gen_device, poison=poison)
    dev_case = case.to("cuda")
    cpu_case = case.to("cpu")
    out, lse, info, flags = run_hip(dev_case, num_splits)
    say("  plan", info, "flags", flags)
    assert flags == 0, "device flags %d on valid input" % flags
    ref_out, ref_lse, secs = oracle_of(cpu_case, batches, kv_heads)
    say("  oracle %.2fs" % secs)
    compare(out, lse, ref_out, ref_lse, sp.name)
    return out, lse, info
