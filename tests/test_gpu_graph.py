"""rattn_decode and rattn_decode_static captured in a HIP graph on a non-default stream.

The header says a call can be captured: it never synchronises the host and allocates
nothing. Each graph holds one call whose plan splits the keys, so the capture records
the split kernel and the combine. The graph is replayed several times, with the inputs
rewritten in place and eager library work and synchronisations between replays, and
every replay must equal (bit for bit) an eager call on the same inputs, which in turn is
checked against the oracle.
"""

import dataclasses

import pytest
import torch

from decode_attention_verify_amd import binding, synth
from tests.parity import compare, oracle_of, say

pytestmark = pytest.mark.gpu


def _case(base, seed, **kw):
    sp = dataclasses.replace(synth.spec(base), **kw)
    return synth.make_case(sp, seed=seed, device="cuda", poison=True)


def _fresh_inputs(case, seed):
    """New q and bias drawn into the case's own buffers (the graph reads those)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    case.q.copy_(torch.randn(case.q.shape, generator=g, device="cuda").to(torch.bfloat16))
    finite = torch.isfinite(case.bias)
    new = 0.5 * torch.randn(case.bias.shape, generator=g, device="cuda")
    case.bias.copy_(torch.where(finite, new, case.bias))


@pytest.mark.parametrize("entry", ["plan", "static"])
@pytest.mark.parametrize("base,kw", [
    ("full_100k", dict(seq_len=20000, dmax=25000, name="graph_decode")),   # per-unit pieces
    ("verify_b16", dict(batch=4, seq_len=("loguniform", 3000, 20000),      # even shares
                        dmax=25000, name="graph_verify")),
])
def test_captured_call_replays_like_eager(entry, base, kw):
    case = _case(base, seed=5, **kw)
    sp = case.spec
    prob = binding.problem_from_case(case)
    shape = (sp.batch, sp.n_rows, sp.num_q_heads)
    out_g = torch.empty(shape + (sp.head_dim,), dtype=torch.bfloat16, device="cuda")
    lse_g = torch.empty(shape, dtype=torch.float32, device="cuda")
    out_e, lse_e = torch.empty_like(out_g), torch.empty_like(lse_g)
    args = (case.q, case.k_cache, case.v_cache, case.k_scale, case.v_scale, case.page_table,
            case.seq_lens, case.bias)
    plan = binding.Plan(prob)
    info = plan.info.as_dict()
    say("graph %s %s plan %s" % (entry, sp.name, info))
    assert info["combine_blocks"] > 0, "the captured call should include the combine"

    def call(out, lse):
        if entry == "plan":
            plan.decode(*args, out, lse)
        else:
            binding.rattn_decode_static(prob, *args, out, lse)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        call(out_g, lse_g)                     # a call before capture, on the same stream
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        call(out_g, lse_g)
    torch.cuda.synchronize()

    cpu = case.to("cpu")
    for rep in range(4):
        _fresh_inputs(case, seed=100 + rep)
        torch.cuda.synchronize()
        call(out_e, lse_e)                     # eager, on the current stream
        torch.cuda.synchronize()
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        say("  replay %d: bitwise equal to eager: %s" % (
            rep, bool(torch.equal(out_g, out_e) and torch.equal(lse_g, lse_e))))
        assert torch.equal(out_g, out_e) and torch.equal(lse_g, lse_e), "replay %d" % rep
        if rep in (0, 3):
            cpu.q.copy_(case.q.cpu())
            cpu.bias.copy_(case.bias.cpu())
            ref, ref_lse, _ = oracle_of(cpu, kv_heads=[1])
            compare(out_g, lse_g, ref, ref_lse, "graph replay %d" % rep)
    assert plan.debug_flags() == 0
    plan.close()
    del graph
