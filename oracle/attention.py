"""The attention definition in float64, with the score matrix materialised.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed: softmax(Q K^T / sqrt(d)) V for Q, K, V of shape (n, d)
per head ("Chapter 3.1 - The Cost of Attention", section 2). Softmax takes the
row maximum for stability and the row sum for normalisation (grasp.study
efficient-attention lesson, "Online Softmax"). The scale is whatever float the
caller passes; the conventional value is 1/sqrt(d).

Readings where the pages are silent (each listed in the design notes):
  * layout: Q, O are [B, H, Nq, d]; K, V are [B, Hkv, Nk, d]; LSE is [B, H, Nq].
  * GQA: query heads are split into Hkv contiguous groups of G = H / Hkv heads,
    each sharing one K/V head ("Quadratic Complexity Bottleneck", GQA entry),
    so query head h reads K/V head h // G. MQA is Hkv = 1 (MQA entry).
  * causal alignment: query row i sits at absolute position p_i = i + Nk - Nq
    (bottom-right), the only alignment under which a one-token decode sees the
    whole KV cache ("Quadratic Complexity Bottleneck", KV cache entry).
  * sliding window W > 0: W keys to the left plus the key itself, j in
    [p - W, p] when causal; |p - j| <= W when not ("Quadratic Complexity
    Bottleneck", sliding-window entry: W tokens to the left and right).
  * LSE = m + ln(l), natural log, over the scaled scores.
  * a row with no visible key gives O = 0 and LSE = -inf.
"""

from __future__ import annotations

import numpy as np

_ROW_BLOCK_ELEMS = 1 << 25  # 256 MiB of float64 scores per block


def _f64(x) -> np.ndarray:
    """Exact widening of a torch tensor (bf16/fp32) or array to float64."""
    try:
        import torch  # local import: the oracle itself needs only numpy
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def visible_mask(Nq: int, Nk: int, causal: bool, window: int, rows=None) -> np.ndarray:
    """Boolean [len(rows), Nk]: may query row i attend to key j?

    Integer logic only. ``rows`` defaults to all Nq rows.
    """
    i = np.arange(Nq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    p = (i + (Nk - Nq))[:, None]          # absolute query positions
    j = np.arange(Nk, dtype=np.int64)[None, :]
    vis = np.ones((p.shape[0], Nk), dtype=bool)
    if causal:
        vis &= j <= p
    if window > 0:
        vis &= j >= p - window
        if not causal:
            vis &= j <= p + window
    return vis


def _head_rows(qh, kh, vh, scale, vis):
    """O and LSE for one head over the given query rows (full key range).

    qh [r, d], kh/vh [Nk, d], vis [r, Nk]. Returns (O [r, d], LSE [r], P [r, Nk]).
    """
    s = scale * (qh @ kh.T)               # the full score matrix for these rows
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)                     # row maximum, -inf for an empty row
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp(s - m_safe[:, None])       # exp(-inf) = 0 on masked entries
    l = p.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    prob = p / l_safe[:, None]
    o = prob @ vh
    lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    o[empty] = 0.0
    return o, lse, prob


def softmax_probs(q, k, scale: float, causal: bool = False, window: int = 0,
                  b: int = 0, h: int = 0, Hkv: int | None = None) -> np.ndarray:
    """The probability matrix P [Nq, Nk] of one head (rows of visible keys sum to 1)."""
    q64, k64 = _f64(q), _f64(k)
    H, Nq, d = q64.shape[1:]
    Hkv = k64.shape[1] if Hkv is None else Hkv
    Nk = k64.shape[2]
    kvh = h // (H // Hkv)
    vis = visible_mask(Nq, Nk, causal, window)
    dummy_v = np.zeros((Nk, 1))
    _, _, prob = _head_rows(q64[b, h], k64[b, kvh], dummy_v, float(scale), vis)
    return prob


def attention_ref(q, k, v, scale: float, causal: bool = False, window: int = 0):
    """Full attention: returns (O [B,H,Nq,d] float64, LSE [B,H,Nq] float64).

    q [B,H,Nq,d], k/v [B,Hkv,Nk,d], any float dtype (widened exactly).
    """
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, H, Nq, d = q64.shape
    Hkv, Nk = k64.shape[1], k64.shape[2]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    G = H // Hkv
    scale = float(scale)
    o = np.zeros((B, H, Nq, v64.shape[3]))
    lse = np.zeros((B, H, Nq))
    rb = max(1, _ROW_BLOCK_ELEMS // max(Nk, 1))
    for r0 in range(0, Nq, rb):
        rows = np.arange(r0, min(Nq, r0 + rb))
        vis = visible_mask(Nq, Nk, causal, window, rows)
        for b in range(B):
            for h in range(H):
                kvh = h // G
                ob, lb, _ = _head_rows(q64[b, h, rows], k64[b, kvh], v64[b, kvh], scale, vis)
                o[b, h, rows] = ob
                lse[b, h, rows] = lb
    return o, lse


def attention_rows_ref(q, k, v, scale: float, causal: bool, window: int,
                       b: int, h: int, rows):
    """Selected query rows of one (b, h), each against every key.

    ``q`` may be the full [B,H,Nq,d] tensor or only row slices are read; K/V are
    read only for head h // G. Returns (O [r, d], LSE [r]) in float64.
    """
    H, Nq = q.shape[1], q.shape[2]
    Hkv, Nk = k.shape[1], k.shape[2]
    kvh = h // (H // Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    qh = _f64(q[b, h][rows])
    kh, vh = _f64(k[b, kvh]), _f64(v[b, kvh])
    vis = visible_mask(Nq, Nk, causal, window, rows)
    o, lse, _ = _head_rows(qh, kh, vh, float(scale), vis)
    return o, lse


def decode_ref(q, k_cache, v_cache, scale: float, window: int = 0):
    """One-token decode: q [B,H,d] against caches [B,Hkv,Nk,d].

    The new token's own K/V are already in the cache, so it is the query at
    the last position Nk - 1 ("Quadratic Complexity Bottleneck", KV cache
    entry). Returns (O [B,H,d], LSE [B,H]) in float64.
    """
    q64 = _f64(q)
    o, lse = attention_ref(q64[:, :, None, :], k_cache, v_cache, scale,
                           causal=True, window=window)
    return o[:, :, 0, :], lse[:, :, 0]


def decode_rows_ref(q, k_cache, v_cache, scale: float, window: int, b: int, heads):
    """Decode output for chosen heads of one sequence b (caches read only for b)."""
    q64 = _f64(q[b])                      # [H, d]
    H = q64.shape[0]
    Hkv, Nk = k_cache.shape[1], k_cache.shape[2]
    G = H // Hkv
    out_o, out_l = [], []
    vis = visible_mask(1, Nk, True, window)
    cache = {}
    for h in heads:
        kvh = h // G
        if kvh not in cache:
            cache[kvh] = (_f64(k_cache[b, kvh]), _f64(v_cache[b, kvh]))
        kh, vh = cache[kvh]
        o, lse, _ = _head_rows(q64[h:h + 1], kh, vh, float(scale), vis)
        out_o.append(o[0])
        out_l.append(lse[0])
    return np.stack(out_o), np.array(out_l)
