"""rattn_decode and rattn_decode_static captured in a HIP graph on a non-default stream.

The header says a call can be captured: it never synchronises the host and allocates
nothing. The graphs hold one call whose plan splits the keys (the split kernel and the
combine), one call of the chunked-prefill kernel, and a whole decode step: the new
tokens' K/V appended to the paged cache (rattn_append_kv), then the layer's attention
over them. Each graph is replayed several times, with the inputs rewritten in place and
eager library work and synchronisations between replays, and every replay must equal
(bit for bit) an eager call on the same inputs, which in turn is checked against the
oracle.
"""

import dataclasses

import pytest
import torch

from decode_attention_verify_amd import binding, synth
from tests.parity import compare, oracle_of, say
from tests.test_gpu_append import _from_codes, _new_rows, _oracle_append

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
    ("prefill_8x2k", dict(batch=1, n_rows=300, seq_len=3000, max_seq_len=3000,   # prefill
                          dmax=3000, name="graph_prefill")),
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
    if info["kernel"] == binding.RATTN_KERNEL_PREFILL:
        assert info["combine_blocks"] == 0
    else:
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


@pytest.mark.parametrize("fmt", [synth.KV_BF16, synth.KV_FP8])
def test_captured_append_and_decode(fmt):
    # one decode step as a serving loop would capture it: the n new tokens of each
    # sequence written into the paged cache, then the attention over the cache
    case = _case("full_100k", seed=41, batch=3, n_rows=4, kv_format=fmt, page_size=64,
                 seq_len=("uniform", 200, 1500), dmax=2000, name="graph_append_decode")
    sp = case.spec
    cpu0 = case.to("cpu")                       # the cache before any append
    prob = binding.problem_from_case(case)
    shape = (sp.batch, sp.n_rows, sp.num_q_heads)
    out_g = torch.empty(shape + (sp.head_dim,), dtype=torch.bfloat16, device="cuda")
    lse_g = torch.empty(shape, dtype=torch.float32, device="cuda")
    out_e, lse_e = torch.empty_like(out_g), torch.empty_like(lse_g)
    k_new, v_new = _new_rows(sp.batch, sp.n_rows, sp.num_kv_heads, sp.head_dim, seed=42)
    kd, vd = k_new.cuda(), v_new.cuda()
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    plan = binding.Plan(prob)
    say("graph append+decode %s plan %s" % (fmt, plan.info.as_dict()))

    def step(out, lse):
        binding.rattn_append_kv(prob, kd, vd, case.page_table, case.seq_lens, case.k_cache,
                                case.v_cache, case.k_scale, case.v_scale, flags)
        plan.decode(case.q, case.k_cache, case.v_cache, case.k_scale, case.v_scale,
                    case.page_table, case.seq_lens, case.bias, out, lse)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step(out_g, lse_g)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step(out_g, lse_g)
    torch.cuda.synchronize()

    for rep in range(3):
        g = torch.Generator().manual_seed(200 + rep)
        k_new = torch.randn(k_new.shape, generator=g).to(torch.bfloat16)
        v_new = torch.randn(v_new.shape, generator=g).to(torch.bfloat16)
        kd.copy_(k_new)
        vd.copy_(v_new)
        _fresh_inputs(case, seed=300 + rep)
        torch.cuda.synchronize()
        step(out_e, lse_e)                      # eager, on the current stream
        torch.cuda.synchronize()
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(out_g, out_e) and torch.equal(lse_g, lse_e))
        say("  replay %d: bitwise equal to eager: %s" % (rep, same))
        assert same, "replay %d" % rep
        if rep in (0, 2):
            # the oracle appends the same rows to the cache as it was before any append
            ok, ov, oks, ovs = _oracle_append(cpu0, k_new, v_new)
            ref_case = dataclasses.replace(
                cpu0, q=case.q.cpu(), bias=case.bias.cpu(), k_cache=_from_codes(ok),
                v_cache=_from_codes(ov), k_scale=None if oks is None else torch.from_numpy(oks),
                v_scale=None if ovs is None else torch.from_numpy(ovs))
            ref, ref_lse, _ = oracle_of(ref_case)
            compare(out_g, lse_g, ref, ref_lse, "graph append+decode replay %d" % rep)
    assert int(flags.item()) == 0
    assert plan.debug_flags() == 0
    plan.close()
    del graph
