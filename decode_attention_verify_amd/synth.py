"""Seeded synthetic inputs for relative-position GQA decode/verify attention.

This module only draws and lays out inputs; it holds none of the attention
arithmetic. Both the HIP path (through the tests and the benchmark) and the CPU
oracle (through the tests) read the tensors it returns.

Shapes follow the pages' workloads:

* page 1 ("vLLM supports Inkling 2 Small", model table): 48 query / 8 KV heads,
  head size 128, a sliding window of 1,024 keys, 7 draft tokens per step;
* page 1 (section on vLLM's optimisations): batch-1 decode at 100K context;
* page 1 (agentic workload table): 32K-256K sessions;
* page 2 ("vLLM TML Inkling support", introduction): context up to 1M tokens;
* page 2 (roadmap) and page 3 (support section): an FP8 KV cache.

Draw order (one seeded ``torch.Generator``): seq_lens, page permutation, q, K, V,
bias. q/K/V are drawn N(0, 1) in float32 and rounded to bfloat16; for the FP8
cache each (token, KV head) vector is quantised with scale ``absmax / 448`` to OCP E4M3
by torch's float8_e4m3fn cast (round to nearest even, after clamping to +-448). The
bias table is ``0.5 * N(0, 1)`` plus an optional linear decay ``-decay * distance``.

The cache is ``[num_pages][Hkv][page_size][D]``: each (page, KV head) block is
contiguous. Logical pages of all sequences are mapped to a random permutation of the
physical pages. With ``poison=True`` every byte the method must never read holds NaN:
unused slots of the last page of each sequence, one spare page, unused page-table
entries (which point at that spare page) and bias columns beyond the largest distance
any query can reach.
"""

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

KV_BF16 = "bf16"
KV_FP8 = "fp8_e4m3"
FP8_MAX = 448.0


@dataclass(frozen=True)
class Spec:
    """A workload shape. ``seq_len`` is an int, or ("uniform"|"loguniform", lo, hi)."""

    name: str
    batch: int
    n_rows: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    window: int
    dmax: int
    page_size: int
    kv_format: str
    seq_len: object
    bias_decay: float = 0.0
    permute_pages: bool = True
    max_seq_len: Optional[int] = None   # planning bound; defaults to the spec's upper bound
    rows_seed: Optional[int] = None     # if set: rows per sequence drawn in [1, n_rows]

    def seq_len_bound(self):
        if self.max_seq_len is not None:
            return int(self.max_seq_len)
        if isinstance(self.seq_len, int):
            return self.seq_len
        return int(self.seq_len[2])


def _named_specs():
    """The five workload families (seed 0 unless stated otherwise)."""
    return {
        # batch 1, 1 row, 6 query / 1 KV head, context 2048, contiguous K/V
        "tiny": Spec("tiny", 1, 1, 6, 1, 128, 0, 2047, 16, KV_BF16, 2048,
                     permute_pages=False),
        # sliding-window layers (W = 1024), seq_lens uniform in [2K, 32K]
        "window_b1": Spec("window_b1", 1, 1, 48, 8, 128, 1024, 1024, 16, KV_BF16,
                          ("uniform", 2048, 32768)),
        "window_b16": Spec("window_b16", 16, 1, 48, 8, 128, 1024, 1024, 16, KV_BF16,
                           ("uniform", 2048, 32768)),
        "window_b64": Spec("window_b64", 64, 1, 48, 8, 128, 1024, 1024, 16, KV_BF16,
                           ("uniform", 2048, 32768)),
        # the sliding-window layers during an 8-row verify step
        "window_verify_b16": Spec("window_verify_b16", 16, 8, 48, 8, 128, 1024, 1031, 16,
                                  KV_BF16, ("uniform", 2048, 32768)),
        # full-context layer, batch 1, 100,000 keys
        "full_100k": Spec("full_100k", 1, 1, 48, 8, 128, 0, 131071, 16, KV_BF16, 100000,
                          bias_decay=1e-5),
        # speculative verify: 8 rows per sequence, batch 16, 32K-256K log-uniform
        "verify_b16": Spec("verify_b16", 16, 8, 48, 8, 128, 0, 262143, 16, KV_BF16,
                           ("loguniform", 32768, 262144), bias_decay=1e-5),
        # a single user's speculative step at 100K context: 4 rows (page 1: about 3.5
        # tokens accepted per step), 24 packed rows per (sequence, KV head)
        "verify4_100k": Spec("verify4_100k", 1, 4, 48, 8, 128, 0, 131071, 16, KV_BF16,
                             100000, bias_decay=1e-5),
        # the same step with two drafts (3 rows: 18 packed rows per (sequence, KV head))
        "verify3_b16": Spec("verify3_b16", 16, 3, 48, 8, 128, 0, 262143, 16, KV_BF16,
                            ("loguniform", 32768, 262144), bias_decay=1e-5),
        # FP8 cache at 1M context, page 64
        "fp8_1m": Spec("fp8_1m", 1, 1, 48, 8, 128, 0, 1048575, 64, KV_FP8, 1048576),
        # batched full-context layers over an FP8 cache (page 64): decode and verify
        "decode_b16_fp8": Spec("decode_b16_fp8", 16, 1, 48, 8, 128, 0, 262143, 64, KV_FP8,
                               ("loguniform", 32768, 262144), bias_decay=1e-5),
        "verify_b16_fp8": Spec("verify_b16_fp8", 16, 8, 48, 8, 128, 0, 262143, 64, KV_FP8,
                               ("loguniform", 32768, 262144), bias_decay=1e-5),
        "verify3_b16_fp8": Spec("verify3_b16_fp8", 16, 3, 48, 8, 128, 0, 262143, 64, KV_FP8,
                                ("loguniform", 32768, 262144), bias_decay=1e-5),
        # the 3-row step over short contexts (the planning bound below 8,192 keys)
        "verify3_b16_8k": Spec("verify3_b16_8k", 16, 3, 48, 8, 128, 0, 8191, 16, KV_BF16,
                               ("loguniform", 2048, 8191), bias_decay=1e-5),
        # the previous model generation's layer shapes (page 1, model table, Inkling
        # column: full layers 64 query / 8 KV heads, sliding layers 64 / 16 with a window
        # of 512; page 2, model architecture: up to 9 tokens per step with MTP heads)
        "v1_full_decode": Spec("v1_full_decode", 1, 1, 64, 8, 128, 0, 131071, 16, KV_BF16,
                               100000, bias_decay=1e-5),
        "v1_window_decode": Spec("v1_window_decode", 16, 1, 64, 16, 128, 512, 512, 16,
                                 KV_BF16, ("uniform", 2048, 32768)),
        "v1_full_verify": Spec("v1_full_verify", 4, 8, 64, 8, 128, 0, 262143, 16, KV_BF16,
                               ("loguniform", 32768, 262144), bias_decay=1e-5),
        "v1_window_verify": Spec("v1_window_verify", 16, 9, 64, 16, 128, 512, 520, 16,
                                 KV_BF16, ("uniform", 2048, 32768)),
        # its full layers during a 9-token step (8 chained MTP heads): 72 packed rows per
        # (sequence, KV head)
        "v1_full_mtp9": Spec("v1_full_mtp9", 4, 9, 64, 8, 128, 0, 262143, 16, KV_BF16,
                             ("loguniform", 32768, 262144), bias_decay=1e-5),
        # the same step when each sequence verifies its own number of tokens, 1..9
        "v1_full_mtp9_varlen": Spec("v1_full_mtp9_varlen", 4, 9, 64, 8, 128, 0, 262143, 16,
                                    KV_BF16, ("loguniform", 32768, 262144), bias_decay=1e-5,
                                    rows_seed=12),
        # one GPU's share of the headline layer under tensor parallelism over KV heads:
        # TP4 keeps 2 KV heads and their 12 query heads, TP8 one and its 6
        "tp4_100k": Spec("tp4_100k", 1, 1, 12, 2, 128, 0, 131071, 16, KV_BF16, 100000,
                         bias_decay=1e-5),
        "tp8_100k": Spec("tp8_100k", 1, 1, 6, 1, 128, 0, 131071, 16, KV_BF16, 100000,
                         bias_decay=1e-5),
        # chunked prefill: 8 chunks of 2048 tokens at about 100K context (page 3, section
        # on coding agents speeding up the implementation)
        "prefill_8x2k": Spec("prefill_8x2k", 8, 2048, 48, 8, 128, 0, 131071, 16, KV_BF16,
                             100000, bias_decay=1e-5),
        # the same chunks over an E4M3 cache (page 2's roadmap: FP8 global attention)
        "prefill_8x2k_fp8": Spec("prefill_8x2k_fp8", 8, 2048, 48, 8, 128, 0, 131071, 64,
                                 KV_FP8, 100000, bias_decay=1e-5),
        # chunks on the previous generation's layer shapes (64q heads): 8-head groups (64/8)
        # and 4-head groups (64/16), 4 chunks of 2048 tokens at 32K
        "prefill_4x2k_g8": Spec("prefill_4x2k_g8", 4, 2048, 64, 8, 128, 0, 131071, 16,
                                KV_BF16, 32768, bias_decay=1e-5),
        "prefill_4x2k_g4": Spec("prefill_4x2k_g4", 4, 2048, 64, 16, 128, 0, 131071, 16,
                                KV_BF16, 32768, bias_decay=1e-5),
        # verify where each sequence checks its own number of drafts, 1..8 (page 3,
        # adaptive verification)
        "verify_b16_varlen": Spec("verify_b16_varlen", 16, 8, 48, 8, 128, 0, 262143, 16,
                                  KV_BF16, ("loguniform", 32768, 262144), bias_decay=1e-5,
                                  rows_seed=11),
    }


SPECS = _named_specs()


def spec(name, **overrides):
    """A named spec, optionally with fields replaced (smaller shapes for tests)."""
    return replace(SPECS[name], **overrides)


@dataclass
class Case:
    spec: Spec
    seed: int
    q: torch.Tensor                    # bf16 [B][n][Hq][D]
    k_cache: torch.Tensor              # bf16 or uint8 (E4M3 codes) [P][Hkv][S][D]
    v_cache: torch.Tensor
    k_scale: Optional[torch.Tensor]    # fp32 [P][Hkv][S] (FP8 only)
    v_scale: Optional[torch.Tensor]
    page_table: torch.Tensor           # int32 [B][max_pages_per_seq]
    seq_lens: torch.Tensor             # int32 [B]
    bias: torch.Tensor                 # fp32 [Hq][dmax+1]
    softmax_scale: float
    max_seq_len: int
    extra: dict = field(default_factory=dict)

    @property
    def num_pages(self):
        return int(self.k_cache.shape[0])

    def to(self, device):
        def mv(t):
            return None if t is None else t.to(device)
        return replace(self, q=mv(self.q), k_cache=mv(self.k_cache), v_cache=mv(self.v_cache),
                       k_scale=mv(self.k_scale), v_scale=mv(self.v_scale),
                       page_table=mv(self.page_table), seq_lens=mv(self.seq_lens),
                       bias=mv(self.bias))


def _draw_seq_lens(sp, gen, device):
    B = sp.batch
    if isinstance(sp.seq_len, int):
        return torch.full((B,), sp.seq_len, dtype=torch.int64)
    kind, lo, hi = sp.seq_len
    if kind == "uniform":
        return torch.randint(lo, hi + 1, (B,), generator=gen, device=device).cpu()
    if kind == "loguniform":
        u = torch.rand((B,), generator=gen, device=device, dtype=torch.float64).cpu()
        vals = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
        return torch.clamp(torch.round(vals), lo, hi).to(torch.int64)
    raise ValueError("unknown seq_len kind %r" % kind)


def _quantise_e4m3(x):
    """x fp32 [..][D] -> (uint8 codes [..][D], fp32 scales [..]) with scale absmax/448."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    y = torch.clamp(x / scale[..., None], -FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.to(torch.float32)


def make_case(sp, seed=0, device="cpu", poison=True, chunk_tokens=1 << 17):
    """Draw one seeded input for spec ``sp`` on ``device`` (CPU or GPU generator)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B, n, Hq, Hkv, D, S = (sp.batch, sp.n_rows, sp.num_q_heads, sp.num_kv_heads,
                           sp.head_dim, sp.page_size)
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    seq_lens = _draw_seq_lens(sp, gen, device)
    bound = sp.seq_len_bound()
    if int(seq_lens.max()) > bound or int(seq_lens.min()) < n:
        raise ValueError("drawn seq_lens fall outside [n, bound]")
    max_pages = -(-bound // S)
    pages_per_seq = [-(-int(L) // S) for L in seq_lens.tolist()]
    used_pages = sum(pages_per_seq)
    spare = used_pages                        # one spare page that nothing may read
    P = used_pages + 1

    if sp.permute_pages:
        perm = torch.randperm(used_pages, generator=gen, device=device).cpu()
    else:
        perm = torch.arange(used_pages)

    q = torch.randn((B, n, Hq, D), generator=gen, device=device).to(torch.bfloat16)

    fp8 = sp.kv_format == KV_FP8
    cache_dtype = torch.uint8 if fp8 else torch.bfloat16
    k_cache = torch.empty((P, Hkv, S, D), dtype=cache_dtype, device=device)
    v_cache = torch.empty((P, Hkv, S, D), dtype=cache_dtype, device=device)
    k_scale = torch.empty((P, Hkv, S), dtype=torch.float32, device=device) if fp8 else None
    v_scale = torch.empty((P, Hkv, S), dtype=torch.float32, device=device) if fp8 else None
    if poison:
        k_cache.fill_(0x7F if fp8 else float("nan"))
        v_cache.fill_(0x7F if fp8 else float("nan"))
    else:
        k_cache.zero_()
        v_cache.zero_()
    if fp8:
        k_scale.fill_(float("nan") if poison else 1.0)
        v_scale.fill_(float("nan") if poison else 1.0)

    # token t of the flattened (b, j) order -> (b, j) -> (physical page, slot)
    lens = seq_lens.tolist()
    tok_b = torch.repeat_interleave(torch.arange(B), seq_lens)
    starts = torch.cumsum(seq_lens, 0) - seq_lens
    tok_j = torch.arange(int(seq_lens.sum())) - starts[tok_b]
    page_off = torch.tensor([0] + pages_per_seq[:-1], dtype=torch.int64).cumsum(0)
    phys_of_token = perm[page_off[tok_b] + tok_j // S]
    slot_of_token = tok_j % S

    # K then V, each drawn over all tokens in (b, j) order, in chunks, and stored
    T = tok_b.numel()
    for cache, scale in ((k_cache, k_scale), (v_cache, v_scale)):
        for t0 in range(0, T, chunk_tokens):
            t1 = min(T, t0 + chunk_tokens)
            x = torch.randn((t1 - t0, Hkv, D), generator=gen, device=device)
            ph = phys_of_token[t0:t1].to(device)
            sl = slot_of_token[t0:t1].to(device)
            if fp8:
                codes, sc = _quantise_e4m3(x)
                cache[ph, :, sl, :] = codes
                scale[ph, :, sl] = sc
            else:
                cache[ph, :, sl, :] = x.to(torch.bfloat16)
            del x

    bias = 0.5 * torch.randn((Hq, sp.dmax + 1), generator=gen, device=device)
    if sp.bias_decay:
        bias = bias - sp.bias_decay * torch.arange(sp.dmax + 1, device=device,
                                                   dtype=torch.float32)[None, :]
    bias = bias.to(torch.float32)

    page_table = torch.full((B, max_pages), spare, dtype=torch.int32)
    for b in range(B):
        o = int(page_off[b])
        page_table[b, :pages_per_seq[b]] = perm[o:o + pages_per_seq[b]].to(torch.int32)

    if poison:
        max_len = max(lens)
        reach = (sp.window - 1) if sp.window > 0 else (max_len - 1)
        touched = min(reach, sp.dmax)
        if touched + 1 <= sp.dmax:
            bias[:, touched + 1:] = float("nan")

    return Case(spec=sp, seed=seed, q=q, k_cache=k_cache, v_cache=v_cache, k_scale=k_scale,
                v_scale=v_scale, page_table=page_table.to(device),
                seq_lens=seq_lens.to(torch.int32).to(device), bias=bias,
                softmax_scale=1.0 / math.sqrt(D), max_seq_len=bound,
                extra={"spare_page": spare, "pages_per_seq": pages_per_seq})


def varlen_rows(case, rows_per_seq):
    """Packed query rows for a call where sequence b brings rows_per_seq[b] rows (at most
    the case's n): the last rows_per_seq[b] of its drawn rows, laid end to end. Returns
    (q [T][Hq][D] bf16, cu_rows [B+1] int32), on the case's device."""
    n = case.spec.n_rows
    if len(rows_per_seq) != case.spec.batch or any(not 0 <= x <= n for x in rows_per_seq):
        raise ValueError("rows per sequence must lie in [0, %d]" % n)
    parts = [case.q[b, n - x:] for b, x in enumerate(rows_per_seq)]
    q = torch.cat(parts, 0).contiguous()
    cu = torch.tensor([0] + list(rows_per_seq), dtype=torch.int64).cumsum(0)
    return q, cu.to(torch.int32).to(case.q.device)


def draw_rows_per_seq(batch, n_max, seed, allow_zero=True):
    """Seeded rows per sequence, uniform in [0 or 1, n_max]."""
    g = torch.Generator().manual_seed(seed)
    lo = 0 if allow_zero else 1
    return torch.randint(lo, n_max + 1, (batch,), generator=g).tolist()
