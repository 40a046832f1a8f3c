"""MI355X-native fused attention forward (gfx950 HIP kernels behind a C ABI).

``fwd`` / ``fwd_fp8`` / ``fp8_prepare`` / ``block_mask`` call the library in
``libattn.so`` (built by ``tiled_attention_05_amd.build``); the ``attn_*``
functions are the same-named thin wrappers of the C entry points. ``inputs``
holds the seeded synthetic workloads and ``flops`` the mask-adjusted work
counts.
"""
from . import flops, inputs  # noqa: F401
from ._lib import (  # noqa: F401
    BF16, F32, FP8_E4M3, MASK_CAUSAL, MASK_DOC, MASK_NONE, MASK_WINDOW, AttnError, attn_block_mask_build,
    attn_block_mask_bytes, attn_fp8_buffer_bytes, attn_fp8_prepare, attn_fwd, attn_status_string,
    block_mask, fp8_prepare, fp8_unpack, fwd, fwd_fp8, load,
)
