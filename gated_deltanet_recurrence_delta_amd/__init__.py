"""MI355X-native gated delta-rule recurrent core with its gated-RMSNorm tail.

The compute lives in ``libgdn.so`` (hand-written HIP for gfx950, C ABI in
``include/gdn.h``); this package is a thin ctypes binding over it that uses
PyTorch only for device memory and streams.
"""

from .binding import (  # noqa: F401
    gdn_abi_version,
    gdn_chunk_prefill,
    gdn_chunk_prefill_noalloc,
    gdn_conv_prologue,
    gdn_decode_step,
    gdn_decode_tokens,
    gdn_gated_rmsnorm,
    gdn_out_proj,
    gdn_out_proj_workspace_size,
    gdn_quantize_act,
    gdn_prefill_workspace_size,
    gdn_status_str,
    gdn_validate_decode,
    gdn_validate_decode_tokens,
    gdn_validate_out_proj,
    gdn_validate_prefill,
    gdn_validate_prologue,
    gdn_validate_quantize_act,
    gdn_validate_rmsnorm,
)
