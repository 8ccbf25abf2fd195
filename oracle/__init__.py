"""Reference oracle for the WUSH transform -> low-bit quantize -> W4A4 matmul path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, CPU implementation
(numpy / scipy, fp64 unless a step pins fp32) of what the GPU path computes.
Only the test-suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code,
constant table or helper with the HIP library under
``aware_block_transforms_amd/`` and imports nothing from it.

Sources (web pages; cited by page title and section):

* "WUSH" news article (chain.bitekongjian.com): the paragraph on the
  construction (Cholesky factor of the weight data, U and S of an SVD, a
  Hadamard matrix; non-orthogonal; block-diagonal), the paragraph on the
  optimality theory, the paragraph on experiments (MXFP4, NVFP4, INT4 layer
  loss), and the paragraph on the deployment workflow (second moments ->
  Cholesky/SVD per block -> transform activations at inference).
* "WUSH: Near-Optimal Adaptive Transforms for LLM Quantization" (AI Radio
  episode, montaan.com): "Problem Setup and Goal" (the layer loss
  l = ||q(T_W W)^T q(T_X X) - W^T X||^2 / (d_out * batch)) and "The gist"
  (Hadamard backbone times a second-moment component; fused GPU kernel).
* "ITQ3_S" article (ai.866data.com): section "Core technique: FWHT
  pre-rotation" (256-dim Walsh-Hadamard pre-rotation before a 3-bit uniform
  quantizer, inverse transform on load, exact round trip).

Modules:

* ``fp``         exact fp32 FMA emulation; E2M1 / E4M3 / E8M0 / fp16 codecs.
* ``transforms`` Sylvester Hadamard, block moments, Cholesky with damping,
                 eigen-decomposition with a sign rule, T_X / T_W assembly,
                 the first-order proxy loss.
* ``quant``      per-block transform (fp32 FMA chain), MXFP4 / NVFP4 / INT4
                 block quantizers and nibble packing.
* ``gemm``       exact decode + fp64 GEMM of quantized operands; layer loss.
* ``had256``     256-point FWHT pre-rotation, 3-bit codes, decode, GEMV.

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (library routines, closed forms, brute force, invariants).  The
one claim with no pin is the size of the loss reductions the pages report on
real Qwen3 layers (parity unpinned; those layers are not available).
"""

from . import fp, transforms, quant, gemm, had256  # noqa: F401
