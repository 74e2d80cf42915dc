"""Plain fp64 CPU oracle for the rotate-then-quantize block codec and the QJL sketch.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The product library (``kv_cache_quantization_amd``) never imports it,
and this package imports nothing from the product: the two share no code,
tables or constant generators.

Every function is written from the pages' description of the method, in their
order and notation, in float64, with no blocking or fusion:

* ``lloyd_max``  - Lloyd-Max scalar quantizer for N(0,1) (eliza quantization README, PolarQuant,
  "Algorithm in one paragraph"; turbopress 0.4.2 README, "Package layout",
  codebooks computed to a fixed point in float64).
* ``hadamard``   - Sylvester Walsh-Hadamard matrix and the randomized rotation
  R = H.D/sqrt(d) (glq 0.7.2 README, "How it works" item 2; turbopress 0.4.2 README,
  "Package layout", hadamard.py).
* ``codec``      - block quantize / dequantize and the QJL residual stage
  (eliza quantization README, PolarQuant, "Algorithm in one paragraph").
* ``qjl``        - QJL key sketch, the asymmetric inner-product estimator and
  the two-stage estimator (eliza quantization README, QJL, "Algorithm in one paragraph";
  qjl_apply.py, ``_qjl_decode_keys`` for the bit order).
* ``attention``  - decode attention over the quantized cache plus an unquantized recent
  window (eliza quantization README, TurboQuant and Fused TurboQuant; glq 0.7.2 README,
  "Inline-dequant E8 KV").
* ``dense``      - dense random rotation with the Beta-distribution codebook (eliza
  quantization README, TurboQuant, "Algorithm in one paragraph").
* ``numerics``   - IEEE round-to-nearest-even to fp16 / bf16 / fp32 and the
  LSB-first bit packing.

Every function here is pinned by ``tests/test_oracle_*.py`` against values the
pages print, closed forms, textbook identities or brute force.
"""

from . import numerics, lloyd_max, hadamard, codec, qjl, attention, dense  # noqa: F401
