"""CPU fp64 oracle for the routed low-bit MoE expert layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute anything under this directory: only the test suite, the smoke
check and the benchmark's CPU-baseline leg use it.  It shares no code with
the HIP library (no kernels, headers, helpers or tables) and imports nothing
from it; the only code both sides use is the seeded input generator
(``synth``), which draws random numbers and holds none of the method's
arithmetic.

Modules
  ptq      post-training quantization: asymmetric RTN codes, bit-plane LUTs,
           truncated-SVD compensators (the encoding step)
  forward  routing, counting sort, dequantization, compensated linears,
           SwiGLU expert FFN and gate-weighted combine (the evaluation step)
  layer    a lazily quantized layer built from fp16 weights with ``ptq``

Everything is plain numpy in float64, except where the method fixes a storage
precision (fp16 scales, LUT entries and factors; uint8 codes and zeros) —
those values are rounded exactly where the encoding stores them.
"""

from . import ptq, forward, layer  # noqa: F401
