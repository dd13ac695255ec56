"""MI355X-native MoE token permute / unpermute.

The work runs in ``libmoe_permute.so`` (hand-written HIP for gfx950, C ABI in
``include/moe_permute.h``); ``binding`` exposes it to Python with the same
entry-point names.
"""

from .binding import (  # noqa: F401
    MoEError,
    MoEPermuteScratch,
    load_library,
    moe_grouped_gemm_bf16,
    moe_permute,
    moe_permute_local,
    moe_permute_local_workspace_size,
    moe_permute_quant_fp8,
    moe_permute_static_scratch,
    moe_permute_supported,
    moe_permute_workspace_size,
    moe_unpermute,
    moe_unpermute_local,
)
