"""Float64 models of the online-softmax recurrence and the split-K merge.

TEST INFRASTRUCTURE ONLY (see the package docstring).

These are not the oracle's answer; they are independent statements of the
steps the pages describe, used to pin the definition in ``attention``:

* Online softmax (grasp.study efficient-attention lesson, "Online Softmax";
  "Chapter 3.1 - The Cost of Attention", section 5): walk the keys block by
  block, keep a running maximum m and running denominator l per query row,
  and rescale what was accumulated so far whenever the maximum grows. The
  pages state the end result equals the one-shot softmax.
* Split-K over keys for decode ("Attention Research", section 2, the
  FlashDecoding line): each split of the key range gives a normalised partial
  output and its log-sum-exp; the partials combine by their LSE weights. The
  combination rule is the reading adopted where the page names the method
  only: O = sum_s exp(lse_s - LSE) O_s, LSE = ln sum_s exp(lse_s); a split
  with no visible key has lse_s = -inf and weight 0.
"""

from __future__ import annotations

import numpy as np

from .attention import _f64, visible_mask


def online_softmax_model(qh, kh, vh, scale: float, vis, block_sizes):
    """One head, all rows: iterate key blocks of the given sizes.

    qh [Nq, d], kh/vh [Nk, d], vis [Nq, Nk] boolean, block_sizes summing to Nk.
    Returns (O [Nq, dv], LSE [Nq]).
    """
    qh, kh, vh = _f64(qh), _f64(kh), _f64(vh)
    nq = qh.shape[0]
    m = np.full(nq, -np.inf)             # running maximum
    l = np.zeros(nq)                      # running denominator
    acc = np.zeros((nq, vh.shape[1]))     # running un-normalised output
    j0 = 0
    for bs in block_sizes:
        j1 = j0 + bs
        s = scale * (qh @ kh[j0:j1].T)
        s = np.where(vis[:, j0:j1], s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1) if bs > 0 else -np.inf)
        # rows that have seen no visible key yet keep everything at zero
        ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(np.where(np.isfinite(m), m, -np.inf) - ref)
        p = np.exp(s - ref[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ vh[j0:j1]
        m = m_new
        j0 = j1
    assert j0 == kh.shape[0]
    seen = l > 0
    o = np.where(seen[:, None], acc / np.where(seen, l, 1.0)[:, None], 0.0)
    lse = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)
    return o, lse


def split_partials_ref(q, k_cache, v_cache, scale: float, window: int, bounds):
    """Decode partials: for each key range [lo, hi) the normalised O_s and lse_s.

    q [B,H,d], caches [B,Hkv,Nk,d]; bounds is a list of (lo, hi).
    Returns (O_s [B,H,S,d], lse_s [B,H,S]).
    """
    q64, k64, v64 = _f64(q), _f64(k_cache), _f64(v_cache)
    B, H, d = q64.shape
    Hkv, Nk = k64.shape[1], k64.shape[2]
    G = H // Hkv
    vis_all = visible_mask(1, Nk, True, window)[0]
    S = len(bounds)
    o_s = np.zeros((B, H, S, v64.shape[3]))
    lse_s = np.full((B, H, S), -np.inf)
    for b in range(B):
        for h in range(H):
            kvh = h // G
            for si, (lo, hi) in enumerate(bounds):
                vis = vis_all[lo:hi]
                if hi <= lo or not vis.any():
                    continue
                s = scale * (k64[b, kvh, lo:hi] @ q64[b, h])
                s = np.where(vis, s, -np.inf)
                m = s.max()
                p = np.exp(s - m)
                l = p.sum()
                o_s[b, h, si] = (p @ v64[b, kvh, lo:hi]) / l
                lse_s[b, h, si] = m + np.log(l)
    return o_s, lse_s


def merge_ref(o_s, lse_s):
    """Combine partials along axis -2 of o_s / axis -1 of lse_s by LSE weights."""
    o_s, lse_s = _f64(o_s), _f64(lse_s)
    M = lse_s.max(axis=-1)
    empty = ~np.isfinite(M)
    M_safe = np.where(empty, 0.0, M)
    w = np.exp(lse_s - M_safe[..., None])          # -inf partials weigh 0
    wsum = w.sum(axis=-1)
    wsum_safe = np.where(empty, 1.0, wsum)
    o = (w[..., None] * o_s).sum(axis=-2) / wsum_safe[..., None]
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, -np.inf, M_safe + np.log(wsum_safe))
    return o, lse
