"""libmiattn: exact fused attention on one AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libmiattn.so`` built from ``csrc/``;
this package is its thin Python binding (argument marshalling only) plus
host-side work accounting. Importing the package does not load the library;
the first call does, and raises if it has not been built.
"""

from .api import (  # noqa: F401
    MiattnError,
    attn_fwd,
    attn_fwd_fp8,
    attn_fwd_varlen,
    attn_decode,
    attn_decode_splitk_noalloc,
    attn_decode_varlen,
    attn_decode_paged,
    attn_bwd,
    attn_bwd_varlen,
    bwd_workspace_bytes,
    decode_workspace_bytes,
    fwd_tile_counts,
    fwd_varlen_tile_counts,
    fwd_tile_shape,
    library_path,
    load_library,
)
