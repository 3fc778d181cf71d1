"""CPU oracle for relative-position GQA decode/verify attention (test infrastructure).

This package is test infrastructure. Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it. The
product path (the HIP library and its Python binding) never calls it, and it
never calls the product path: the two share no code.

Everything here is plain numpy in float64 (pure Python for ``bruteforce``), written
from the definition of the method:

* page 2 ("vLLM TML Inkling support", section on the model architecture) states that
  the model replaces rotary embeddings with a learned relative-position term that is
  added to the attention logits before the softmax; heads have size 128 and use GQA;
* page 1 ("vLLM supports Inkling 2 Small", model table) gives 48 query / 8 KV heads and
  a sliding window of 1,024 tokens, and (section on trying the model) 7 speculative
  tokens per step, which the target model verifies together;
* page 2 (roadmap) and page 3 ("vLLM supports Reflection Beam", support section) speak
  of an FP8 KV cache.

The pages do not say how the relative term is parameterised. The reading taken here is
a per-query-head float32 table ``B[h][min(i - j, Dmax)]`` indexed by the query-key
distance, added after the ``1/sqrt(d)`` scaling of ``q . k``.

Parity of this oracle is pinned, in ``tests/test_oracle_pins.py``, against library
routines (torch SDPA in float64), closed forms, invariants and brute force. The readings
that the pages leave open (bias after the scale, a window of W keys including the token
itself, verify rows at the last n positions, head h using KV head h div G) are fixed by
the problem statement, not by the pages: parity unpinned by the pages for those choices.
"""

from .formats import bf16_bits_to_f64, e4m3fn_codes_to_f64
from .attention import relative_attention, partial_attention
from .combine import combine_partials
from .bruteforce import bruteforce_attention
from .append import append_kv, e4m3fn_encode, quantise_rows_e4m3
from .varlen import relative_attention_varlen

__all__ = [
    "bf16_bits_to_f64",
    "e4m3fn_codes_to_f64",
    "relative_attention",
    "partial_attention",
    "combine_partials",
    "bruteforce_attention",
    "append_kv",
    "e4m3fn_encode",
    "quantise_rows_e4m3",
    "relative_attention_varlen",
]
