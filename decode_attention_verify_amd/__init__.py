"""rattn: relative-position GQA decode/verify attention for MI355X (gfx950).

The compute path is the HIP library ``librattn.so`` (built from ``csrc/``) behind a
C ABI; ``decode_attention_verify_amd.binding`` is its thin ctypes binding. Importing
this package does not load the library, so the input generator (``synth``) and the
byte accounting (``accounting``) stay usable on machines without a GPU; every call
into the binding loads the library and fails loudly when it is missing.
"""

__all__ = ["synth", "accounting", "binding"]
