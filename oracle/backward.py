"""Gradients of exact attention in float64, score matrices materialised.

TEST INFRASTRUCTURE ONLY (see the package docstring).

For O = softmax(scale * Q K^T + mask) V and an upstream gradient dO, the
gradients of L = sum(O * dO) follow from the chain rule through the product
with V, the row softmax and the scaled product Q K^T:

    P   = softmax(S),  S = scale * Q K^T (masked entries -inf, so P = 0 there)
    dV  = P^T dO
    dP  = dO V^T
    dS  = P * (dP - rowsum(P * dP))          (softmax Jacobian, row by row)
    dQ  = scale * dS K
    dK  = scale * dS^T Q

With GQA, a K/V head's gradient is the sum over the query heads of its
group. The pages call for the backward pass to recompute the attention
matrix instead of storing it ("Quadratic Complexity Bottleneck",
FlashAttention entry; "Chapter 3.1 - The Cost of Attention", section 5);
this oracle simply materialises it, as the definition does.
"""

from __future__ import annotations

import numpy as np

from .attention import _f64, visible_mask


def attention_bwd_ref(q, k, v, do, scale: float, causal: bool = False, window: int = 0,
                      return_terms: bool = False, kv_heads=None):
    """(dq [B,H,Nq,d], dk [B,Hkv,Nk,d], dv [B,Hkv,Nk,d]) in float64.

    With return_terms, also a dict of per-head fp64 intermediates keyed by
    (b, h): "P", "dS" (each [Nq, Nk]) for error bounds in tests.
    kv_heads restricts the work to the query heads of the listed K/V heads
    (the other entries of the results stay 0).
    """
    q64, k64, v64, do64 = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, Nq, d = q64.shape
    Hkv, Nk = k64.shape[1], k64.shape[2]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    G = H // Hkv
    scale = float(scale)
    vis = visible_mask(Nq, Nk, causal, window)
    dq = np.zeros_like(q64)
    dk = np.zeros_like(k64)
    dv = np.zeros_like(v64)
    terms = {}
    heads = range(H) if kv_heads is None else [kh * G + i for kh in kv_heads for i in range(G)]
    for b in range(B):
        for h in heads:
            kvh = h // G
            s = np.where(vis, scale * (q64[b, h] @ k64[b, kvh].T), -np.inf)
            m = s.max(axis=1, initial=-np.inf)
            empty = ~np.isfinite(m)
            p = np.exp(s - np.where(empty, 0.0, m)[:, None])
            l = p.sum(axis=1)
            p = p / np.where(empty, 1.0, l)[:, None]       # rows of no key stay 0
            dP = do64[b, h] @ v64[b, kvh].T
            dS = p * (dP - (p * dP).sum(axis=1)[:, None])
            dq[b, h] = scale * (dS @ k64[b, kvh])
            dk[b, kvh] += scale * (dS.T @ q64[b, h])
            dv[b, kvh] += p.T @ do64[b, h]
            if return_terms:
                terms[(b, h)] = {"P": p, "dS": dS}
    if return_terms:
        return dq, dk, dv, terms
    return dq, dk, dv
