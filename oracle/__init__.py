"""Plain CPU oracle for block-scaled low-bit quantization and the weight-only
quantized matmul y = x . dequant(Wq)^T.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import anything here.  The product path
(the HIP library behind its C ABI and the Python binding over it) never
imports, calls or links this package, and this package shares no code with it.

Arithmetic policy
-----------------
* Exact work is done in fp64 and integer bit operations: fp64 holds every fp32
  and bf16 input exactly, every power-of-two scaling of them, and every product
  of two narrow-format values (E4M3, E2M1, INT4, bf16).
* Where the method names an fp32 operation (the scale amax/448, the division
  x/scale), the oracle performs exactly that IEEE-754 fp32 operation with NumPy
  float32 arithmetic (round to nearest, ties to even).
* Integer rounding uses numpy.rint (round half to even).

Modules
-------
formats   number-format algebra and decode tables (bias, max finite, min normal,
          epsilon; E4M3, E2M1, E8M0, bf16 encode/decode)
e4m3      fp32 -> OCP E4M3 "fn", RNE + satfinite; per-block and per-row scaling
e8m0      the exponent-first 0.75-threshold E8M0 shared-scale rule
mxfp4     E2M1 element rounding and the MXFP4 block quantizer
mx        MX block quantizers under five E8M0 rules (exponent-first with the
          format's rounding increment, threshold 0.5, strict OCP, the old
          reciprocal-multiply rule, the round-up division rule) for E2M1 and E4M3
          elements
nvfp4     NVFP4: E2M1 blocks of 16 with an E4M3 scale and a per-tensor fp32 scale
int4      symmetric INT4 group quantizer with bf16 scales
int4_asym asymmetric INT4: unsigned codes, bf16 group scale, integer zero-point
dequant   packed weights + scales -> bf16 operands
gemm      fp64 reference matmul and the acceptance bound
w8a8      W8A8 FP8: static per-tensor activation quantizer, 128 x 128 weight
          blocks, the block-scaled fp32 reference
w4a8      MoE routing, W4A8 scale recipe, INT4 -> E4M3 lookup table, grouped GEMM

Parity status: every function is pinned by CPU tests against values the pages
print, closed forms, library routines (torch CPU casts) or brute force, except
the nibble order inside a byte / word (pack and unpack), which the pages do not
fix: parity unpinned (self-consistency only).
"""
