"""CPU oracle for the QUADS rollout hot path -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct NumPy (fp64) statement of what
the GPU library computes.  It exists to check the HIP kernels, nothing else:
only the test-suite, the smoke check of the graft entry point and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the
``nvfp4_w4a4_quantized_act_amd`` package and its C-ABI library) never imports,
links or calls anything in here, and this package imports nothing from it.

Source of the method: "QUADS: Stabilizing NVFP4 Reinforcement Learning for MoE
via QUantization-error Alignment across Dual Sides" (arXiv 2607.15810):
  * section 2.2, "FP4" paragraph -- NVFP4: E2M1 core with magnitudes
    {0, 0.5, 1, 1.5, 2, 3, 4, 6}, 16-element blocks sharing an E4M3 scale, an
    optional per-tensor FP32 scale;
  * section 2.2, "FP8" paragraph -- E4M3 with maximum magnitude 448;
  * section 3.1, Eq. (6), (7), (9) -- the layer product, weight QDQ and
    activation QDQ;
  * section 3.3, Eq. (20)-(24) -- residual, targeted compensation, channel
    score and top-k selection (Residual Activation Compensation, RAC).

Where the pages leave a step open, the reading taken is stated in the module
that implements it.

Modules:
  formats -- E2M1/E4M3/bf16/fp32 encodings and exact round-to-nearest-even
  nvfp4   -- tensor scale, block scale, element codes, pack/unpack, dequant
  rac     -- residual, fixed-order channel score, top-k, second pass
  moe     -- token packing, grouped W4A4 GEMM with compensation, SwiGLU,
             combine
"""

from . import formats, nvfp4, rac, moe  # noqa: F401
