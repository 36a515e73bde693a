"""Plain CPU oracle for the quantized rollout linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
anything in this package: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library and imports
nothing from it.

What it computes (each module cites the passage it follows):

* ``codecs``  -- the E2M1 (FP4) and OCP E4M3 (FP8) value grids and their
  round-to-nearest-even, saturating encoders, written as a nearest-value search
  over the grid.
* ``nvfp4``   -- the NVFP4 weight quantizer (E2M1 codes, 16-element blocks along
  K, one E4M3 scale per block, one FP32 tensor scale).
* ``fp8``     -- the blockwise FP8 recipe: E4M3 codes with one FP32 scale per
  128x128 weight tile and per 1x128 activation segment, and its variant with
  power-of-two (E8M0) scales.
* ``gemm``    -- the rollout linear layer y = x . dequant(Wq)^T + s (x A^T) B^T
  as its plain definition in float64.
* ``requant`` -- the whole-policy requantization: the per-tensor quantizers
  applied to every tensor of a list.
* ``update``  -- a training step's dense bf16 update applied to the weights, followed by
  that requantization.
* ``kvcache`` -- the FP8 KV-cache codec: E4M3 codes with one float32 scale per cached
  (token, head) vector, scattered to and gathered from cache slots.
* ``backward`` -- the layer's backward pass with the NVFP4 base frozen: dX through the
  dequantized weight and the adapter, and the adapter's gradients dA, dB, in float64.

Quantizer arithmetic is IEEE float32 with round-to-nearest-even, because that is
where the codes are decided and the GPU decides them in float32 too; every
GEMM and every dequantized value is float64.
"""

from . import codecs, nvfp4, fp8, gemm, requant, update, kvcache, backward  # noqa: F401
