"""Plain, slow CPU oracle of the DCKV prompt-KV-cache codec (test infrastructure).

This package is test infrastructure.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The HIP library
(``learned_kv_cache_dckv_amd``) never imports it and shares no code with it; the
two meet only through the seeded inputs of ``dckv_synth``.

It follows the DCKV digest page ("DCKV: Learned Transform Coding of the Prompt
KV Cache in Hybrid Language Models", trove.briskstack.com), section "How it
works", and the paper abstract (scholarbro.com page of the same title).  Where
the pages leave a step open, the reading taken is stated in the function that
implements it.  Arithmetic is float64 unless a step names another precision;
bf16 rounding is round-to-nearest-even and happens only at the named points.

Modules:
  bf16    exact float64 <-> bf16 conversion
  plan    steps, dropped components, integer Laplace tables, plan CRC
  rans    interleaved 32-bit rANS: a scalar per-group coder and a lock-step
          vectorised coder over all groups (same format, cross-checked)
  stream  the byte-stream layout (writer and validating parser)
  codec   encode / decode of a request (transform, conditional means,
          checkerboard, quantiser, escapes, correction MLP, RoPE)
"""
from . import bf16, plan, rans, stream, codec  # noqa: F401
