"""CPU oracle for the NVFP4 weight-only Gemma-4-26B-A4B MoE expert block.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, float64 statement of
what the block computes, written from the model-card pages.  It exists to check
the HIP library, never to stand in for it: only the tests, the smoke entry point
and the benchmark's CPU-baseline leg may import it.  It shares no code, table or
constant generator with the HIP path; both sides take their inputs from the
seeded generators in ``moe_synth`` only.

Parts and the passages they follow (page title, section):

* ``formats``  -- E2M1 element values, OCP E4M3 block-scale decoding, the
  two-level NVFP4 dequantisation, nibble packing.  "Gemma-4-26B-A4B-NVFP4-mlx"
  (Quantization recipe table and Notes: E2M1, group 16, E4M3 block scale,
  per-tensor FP32); "gemma-4-26B-A4B - NVFP4A16" (Quantization details).
* ``quantize`` -- the block quantiser S_block = max|w|/V_max, V_max = 6,
  q = clip(round(w/S_block), -6, 6), ŵ = q * S_block.
  "Gemma-4-26B-A4B-it-NVFP4" README (block-quantisation formulas).
* ``moe`` -- router, token bucketing, GELU-tanh gated experts, weighted sum,
  whole block and the dense "over-read" cross-check.
  "Gemma 4 26B-A4B (MoE) - Core AI" (Architecture: block pseudocode and router
  description; Compression recipe: dense over-read; Decode only: sort-by-expert
  grouped GEMM).

Every function's result is pinned by ``tests/test_oracle_*.py`` against
something other than itself (closed forms, torch library routines, brute force,
invariants); functions without such a pin would say "parity unpinned" -- none
currently does.
"""
