"""Seeded synthetic inputs for the 4-bit mixture-of-experts layer.

This module only draws random inputs; it holds none of the layer's arithmetic.
Both the CPU oracle (``oracle/``) and the HIP path draw their inputs from here,
so the two sides always see identical arrays.

Formats (the checkpoint format of the Lily pages: 4-bit affine weights, groups
of 64 along the input dimension, one bf16 scale and one bf16 bias per group):

* a packed code word is a little-endian uint32 holding 8 codes, code ``k`` of a
  row in word ``k // 8`` at bits ``4*(k % 8) .. 4*(k % 8) + 3`` (low nibble
  first).  A uniformly random word is therefore 8 i.i.d. U{0..15} codes.
* projection ``W`` of shape [N][K] (N outputs, K inputs) is stored as codes
  uint32 [N][K/8], scale and bias bf16 bits (uint16) [N][K/64]; routed experts
  stack these as [E][N][...].
* gate and up have N = I, K = H; down has N = H, K = I.
* activations are bf16 bits (uint16) [T][H]; the router weight is stored
  transposed, bf16 [E][H] (one contiguous row per expert).

Distributions: x ~ N(0,1) rounded to bf16; router weight ~ N(0, sigma) with
sigma = 1/sqrt(H), rounded to bf16; scale ~ U(0.002, 0.02) rounded to bf16;
bias = -8 * scale (exact in bf16).  The skewed-routing workload adds a fixed
per-expert logit bias b_e = -s * ln(e + 1), the log of an unnormalised Zipf(s)
prior over expert rank e + 1.  The expert-parallel share workload biases every
expert outside [0, E/n) by -32, so that the picks stay on one GPU's share of the
experts under expert parallelism over n GPUs.
"""
from .inputs import (  # noqa: F401
    LayerInputs,
    Projection,
    WORKLOADS,
    bf16_bits_to_f32,
    ep_share_bias,
    f32_to_bf16_bits,
    make_layer,
    make_projection,
    zipf_bias,
)
