"""CPU oracle for blockwise-scaled FP8 linear-layer training.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code,
header, table or constant generator with the HIP library; the only thing the
two sides have in common is the seeded input generator, which lives in its own
module and holds none of the method's arithmetic.

What it computes (plain numpy, slow on purpose):

* ``e4m3``   -- the OCP FP8 E4M3 ("FN") format: decode table from the format
  definition and a round-to-nearest-even, saturating encoder.
* ``quant``  -- the blockwise quantizers (1x128 rowwise, 1x128 colwise,
  128x128, 3-D colwise), each in a scalar-loop form for small inputs and a
  vectorized form of the same definition.
* ``gemm``   -- the blockwise-scaled matmuls as "dequantize to float64, then
  float64 matmul", dense and grouped, plus the per-element tolerance of the
  parity bar.
* ``swiglu`` -- the gated FFN activation silu(a) * b and its derivative,
  each rounded once to bf16 (what the fused activation-and-quantize kernels
  quantize).
* ``mx``     -- the MXFP8 variant (OCP Microscaling: 32-element blocks, E8M0
  power-of-two scales, E4M3 elements) quantizer and its GEMM.

Sources: the three pytorch/ao pull-request pages on blockwise FP8 training
("[not for land] float8 blockwise scaling training prototype using
deep_gemm", "[mxfp8 moe training] use new 3d colwise quantization kernel",
"add FSDP and TP tests for Float8BlockwiseLinear") and the OCP 8-bit floating
point specification for the E4M3 encoding, which the pages leave unnamed.

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against something other than itself (format closed forms, exact rational
arithmetic, brute force, invariants, torch's own float8 cast).  The one
reading the pages cannot decide -- the block shape of the 3-D colwise
quantizer -- is documented as "parity unpinned" in ``quant.quant_3d_colwise``.
"""

from . import e4m3, quant, gemm, swiglu  # noqa: F401
