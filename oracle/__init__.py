"""CPU oracle for the routed-expert MXFP4 MoE layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
numpy statement of what the layer computes.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import or run it; the GPU
library never does, and the two share no code.

Sources (cited by page and section):
  * txtmix.com article "DeepSeek V4 Flash 单卡 MI300X ..." -- §1 (256 experts,
    top-6; expert weights kept in MXFP4), §3 (MXFP4 = 4-bit values with a shared
    E8M0 scale; the bitmatrix padding-lane mask), §8 (decode is weight-streaming
    bound), §9 (the SwiGLU clamp: gate <= limit, -limit <= up <= limit, applied
    before the product; limit 10 for this checkpoint).
  * aihot.vn README translation, section "Định tuyến MXFP4" (the bitmatrix pads
    its block columns to the kernel block and must mask by the logical size).
  * OCP Microscaling Formats (MX) v1.0 for the E2M1 element and E8M0 scale codes.

Readings where the pages are silent (each also listed in the design notes):
  * route: the k largest logits per token, ordered by (logit descending, expert
    index ascending); -0.0 equals +0.0; weights = softmax over the k chosen logits.
  * gather lists slot ids t*k+j grouped by expert ascending, token ascending
    within an expert; scatter is its inverse permutation.
  * W1 rows [0, I) are the gate half and [I, 2I) the up half.
  * the clamp is off when the limit is <= 0 or not finite.
  * matrix products accumulate in fp32 over the dequantised weights; elementwise
    steps run in fp64.

Pins: every function here is checked by the CPU tests against values the spec
or mathematics fixes (decode tables, brute force on tiny inputs, closed forms,
exact metamorphic identities).  FFN values at full size have no pin beyond the
oracle itself and the identities; that part is "parity unpinned" by the pages.
"""
from .mx import e2m1_decode, e8m0_decode, dequant_mxfp4, E2M1_VALUES
from .moe import (route, bitmatrix, expert_offsets, swiglu, ffn, combine,
                  moe_layer, dense_moe, bf16_to_f32)

__all__ = ["e2m1_decode", "e8m0_decode", "dequant_mxfp4", "E2M1_VALUES", "route",
           "bitmatrix", "expert_offsets", "swiglu", "ffn", "combine", "moe_layer",
           "dense_moe", "bf16_to_f32"]
