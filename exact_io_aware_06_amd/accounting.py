"""Algorithmic work and traffic of the attention path (host-side arithmetic).

These counts price the kernels against the roofline. They are the useful
work only: masked pairs inside boundary tiles, exponentials and other vector
work are not counted as FLOPs, and re-reads served by caches are not counted
as bytes.

* Prefill: every visible (query, key) pair costs one d-long dot product for
  Q K^T and one d-long multiply-add into the output for P V, i.e. 4 d FLOPs.
  The full (non-causal, unwindowed) count 4 d N^2 is the O(n^2 d) cost of the
  QK^T product the pages describe ("Chapter 3.1 - The Cost of Attention",
  section 2; "Quadratic Complexity Bottleneck", compute entry).
* Decode: the KV cache is read once per step ("Attention Research", section 1:
  memory O(S), read every decode step), plus q in and O / LSE out.
"""

from __future__ import annotations


def visible_pairs(Nq: int, Nk: int, causal: bool, window: int) -> int:
    """Number of (query, key) pairs a single head attends over.

    Query row i sits at position p = i + Nk - Nq. It sees keys j in
    [lo, hi] with lo = max(0, p - W) if W > 0 else 0, and hi = p if causal,
    else min(Nk - 1, p + W) if W > 0, else Nk - 1.
    """
    if Nq <= 0 or Nk <= 0:
        return 0
    total = 0
    off = Nk - Nq
    # Rows fall into a few linear regimes; summing per row keeps this obvious.
    for i in range(Nq):
        p = i + off
        lo = max(0, p - window) if window > 0 else 0
        if causal:
            hi = min(Nk - 1, p)
        elif window > 0:
            hi = min(Nk - 1, p + window)
        else:
            hi = Nk - 1
        if hi >= lo:
            total += hi - lo + 1
    return total


def prefill_flops(B: int, H: int, Nq: int, Nk: int, d: int, causal: bool, window: int) -> int:
    """Algorithmic FLOPs of one forward call: 4 d per visible pair per head."""
    return 4 * d * visible_pairs(Nq, Nk, causal, window) * B * H


def dense_attention_ops(n: int, d: int = 1) -> int:
    """Multiply-adds of the full n x n score matrix QK^T: n^2 d."""
    return n * n * d


def score_matrix_bytes(n: int, bytes_per_elem: int = 4) -> int:
    """Bytes of one head's materialised n x n score matrix."""
    return n * n * bytes_per_elem


def prefill_bytes(B, H, Hkv, Nq, Nk, d, elem_bytes=2, lse=True) -> int:
    """Compulsory HBM bytes of one forward call: Q, K, V read once; O (+LSE) written."""
    qo = 2 * B * H * Nq * d * elem_bytes
    kv = 2 * B * Hkv * Nk * d * elem_bytes
    return qo + kv + (B * H * Nq * 4 if lse else 0)


def decode_bytes(B, H, Hkv, Nk, d, elem_bytes=2, window=0, lse=True) -> int:
    """Compulsory HBM bytes of one decode step.

    K and V are read once over the visible keys (all Nk, or the last W + 1
    with a window); q is read and O (and LSE) written once.
    """
    keys = Nk if window <= 0 else min(Nk, window + 1)
    kv = 2 * B * Hkv * keys * d * elem_bytes
    qo = 2 * B * H * d * elem_bytes
    return kv + qo + (B * H * 4 if lse else 0)


def decode_flops(B, H, Nk, d, window=0) -> int:
    keys = Nk if window <= 0 else min(Nk, window + 1)
    return 4 * d * keys * B * H


def packed_visible_pairs(cu_q, cu_k, causal: bool, window: int) -> int:
    """Visible (query, key) pairs of one head over packed documents.

    The mask is block-diagonal by document ("What Lost, and Why", closing
    section: the mask restarts at each document boundary), so the count is
    the sum of each document's own count.
    """
    total = 0
    for e in range(len(cu_q) - 1):
        total += visible_pairs(int(cu_q[e + 1]) - int(cu_q[e]), int(cu_k[e + 1]) - int(cu_k[e]),
                               causal, window)
    return total


def packed_flops(H: int, cu_q, cu_k, d: int, causal: bool, window: int) -> int:
    """Algorithmic FLOPs of one packed forward call: 4 d per visible pair per head."""
    return 4 * d * H * packed_visible_pairs(cu_q, cu_k, causal, window)


def decode_kvlens_bytes(H, Hkv, kv_lens, d, elem_bytes=2, window=0, lse=True) -> int:
    """Compulsory bytes of one decode step over caches of per-sequence length."""
    keys = sum(int(n) if window <= 0 else min(int(n), window + 1) for n in kv_lens)
    B = len(kv_lens)
    kv = 2 * Hkv * keys * d * elem_bytes
    qo = 2 * B * H * d * elem_bytes
    return kv + qo + (B * H * 4 if lse else 0)


def decode_paged_bytes(H, Hkv, kv_lens, d, page_size, elem_bytes=2, window=0, lse=True) -> int:
    """Compulsory bytes of one paged decode step: the keys and values each
    sequence sees, q, O and LSE, plus the block-table entries of its pages."""
    pages = sum(-(-int(n) // page_size) for n in kv_lens)
    return decode_kvlens_bytes(H, Hkv, kv_lens, d, elem_bytes, window, lse) + 4 * pages


def backward_flops(B, H, Nq, Nk, d, causal, window) -> int:
    """Algorithmic FLOPs of one backward call: 10 d per visible pair per head
    (recomputing S, then dP, dV, dK and dQ at 2 d each: 2.5 x the forward)."""
    return 10 * d * visible_pairs(Nq, Nk, causal, window) * B * H


def backward_executed_flops(B, H, Nq, Nk, d, causal, window) -> int:
    """Matrix-core FLOPs the two-kernel backward actually issues: S and dP are
    computed in both the dQ pass and the dK/dV pass, 14 d per visible pair."""
    return 14 * d * visible_pairs(Nq, Nk, causal, window) * B * H
