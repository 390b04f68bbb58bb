"""Fused scaled-dot-product attention forward for MI355X (gfx950).

The compute path is the HIP library ``libattn.so`` built from ``csrc/``; this
package only binds its C ABI (see ``api``) and draws seeded inputs
(``inputs``). Importing the package does not load the library; the first call
does, and raises ImportError if it has not been built.
"""
from .api import (  # noqa: F401
    AttnError,
    attn_fwd,
    attn_fwd_naive,
    attn_fwd_noalloc,
    attn_fwd_plan,
    attn_fwd_splitk,
    attn_fwd_tile_choice,
    attn_fwd_tile_count,
    attn_fwd_tile_info,
    attn_fwd_tiled,
    attn_fwd_workspace_size,
    attn_naive_scratch_size,
    attn_qkv_proj,
    attn_qkv_proj_tiling,
    attn_softmax_rows,
    attn_splitk_workspace_size,
    attn_status_string,
    attn_version,
    load_library,
)
