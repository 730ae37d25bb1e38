"""Plain, slow, obviously-correct CPU attention in float64: the oracle.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's CPU
baseline leg may import anything from here. The HIP library never calls it,
and it shares no code, header, table or helper with the HIP library.

What it computes (exact scaled dot-product attention):

    O = softmax(scale * Q K^T + mask) V,   LSE = row-wise ln sum exp(scores)

as defined in "Chapter 3.1 - The Cost of Attention", section 2 ("Why
self-attention is quadratic, precisely"), with the full score matrix
materialised exactly the way the pages describe the unfused method
("What Lost, and Why", section "Why they lost"). The tiled, fused method
reaches the same result up to rounding ("Chapter 3.1", section 5; the
grasp.study efficient-attention lesson, "Online Softmax"), so the oracle is
the definition, not the tiled algorithm.

Modules:
  attention  - the definition (full score matrix per head), row samples, decode
  online     - the pages' online-softmax recurrence and the split-K merge, as
               independent fp64 models used only to pin the definition
  tiles      - which (query-tile, key-tile) blocks hold any visible pair
  backward   - gradients dq, dk, dv of the definition (chain rule through the
               materialised softmax)
  varlen     - packed documents (block-diagonal mask), decode over caches
               of per-sequence length and over paged caches
"""

from .attention import (  # noqa: F401
    visible_mask,
    softmax_probs,
    attention_ref,
    attention_rows_ref,
    decode_ref,
    decode_rows_ref,
)
from .backward import attention_bwd_ref  # noqa: F401
from .online import online_softmax_model, split_partials_ref, merge_ref  # noqa: F401
from .tiles import tiles_needed  # noqa: F401
from .varlen import (  # noqa: F401
    packed_visible_mask,
    attention_varlen_ref,
    attention_varlen_rows_ref,
    decode_kvlens_ref,
    decode_kvlens_rows_ref,
    decode_paged_ref,
    gather_pages,
)
