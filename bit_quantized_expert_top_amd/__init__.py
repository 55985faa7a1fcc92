"""MI355X (gfx950) mixture-of-experts layer with 4-bit affine expert weights.

Thin Python binding over the C ABI of ``libmoeq4.so`` (``include/moe_q4.h``).
The functions carry the C names (``moe_route``, ``moe_expert_gemm_q4``,
``moe_down_combine``, ``moe_expert_ffn_q4``, ``moe_combine``, ``moe_combine_residual``, ``moe_down_combine_residual``, ``moe_layer``, ``moe_layer_chunked``, ``moe_decode``, ``moe_decode_static``, ``moe_decode_residual``, ``moe_rmsnorm_residual``,
``moe_dequant_q4``, ``moe_query``, ``moe_packed_bytes``; ``moe_pack_weights``
runs inside ``DeviceLayer``); they only check tensors and marshal
pointers: every step of the layer runs in the library's HIP kernels.  PyTorch
provides device memory and the stream.  Loading fails loudly when the library
has not been built (``python -m bit_quantized_expert_top_amd.build`` or
``__graft_entry__.build()``).
"""
from .binding import (  # noqa: F401
    DeviceLayer,
    MoeError,
    Routing,
    Shape,
    UnsupportedWeights,
    lib,
    moe_combine,
    moe_combine_residual,
    moe_decode,
    moe_decode_residual,
    moe_debug_status,
    moe_decode_static,
    moe_dequant_q4,
    moe_down_combine,
    moe_down_combine_residual,
    moe_expert_ffn_q4,
    moe_expert_gemm_q4,
    moe_layer,
    moe_layer_chunked,
    moe_packed_bytes,
    moe_query,
    moe_query_chunked,
    moe_rmsnorm_residual,
    moe_route,
    moe_status_str,
    workspace,
    workspace_chunked,
)
