"""Online-softmax attention for MI355X (gfx950).

The kernels live in libattn.so (C ABI declared in include/attn.h); this
package holds its sources (csrc/), the build step (build.py), the ctypes
binding (binding.py) and the seeded synthetic-input generator (inputs.py).
Importing the package does not load the library; the first call does, and
fails loudly if it has not been built.
"""
from .binding import (  # noqa: F401
    ATTN_BF16,
    ATTN_F32,
    EXPORTS,
    LIB_PATH,
    AttnError,
    attn_abi_version,
    attn_bwd,
    attn_bwd_fused,
    attn_bwd_fused_workspace_bytes,
    attn_bwd_workspace_bytes,
    attn_decode,
    attn_decode_noalloc,
    attn_decode_paged,
    attn_decode_workspace_bytes,
    attn_fwd,
    attn_fwd_tile_override,
    attn_bwd_tile_override,
    attn_bwd_split_workspace_bytes,
    attn_bwd_plan,
    attn_fwd_tile_plan,
    attn_set_timing_events,
    attn_status_str,
    attn_supports,
    lib,
)
