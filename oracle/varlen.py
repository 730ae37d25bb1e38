"""Packed variable-length sequences and per-sequence KV lengths, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Passage followed: when several documents are packed into one training
sequence, the attention mask has to start afresh at every document boundary;
a mask that lets tokens see the previous document is a silent correctness
bug ("What Lost, and Why", the closing section on one more casualty of the
efficiency work).

Readings (the pages give no layout or interface for packing):
  * a packed batch is the concatenation of ``num_seqs`` documents along the
    token axis of one sequence: Q, O are [H, total_q, d], K, V are
    [Hkv, total_k, d], LSE is [H, total_q] (the fixed-length layout with
    B = 1 and the token axis shared by all documents);
  * ``cu_q`` / ``cu_k`` hold num_seqs + 1 non-decreasing row offsets with
    cu[0] = 0 and cu[-1] = total: document e owns query rows
    [cu_q[e], cu_q[e+1]) and key rows [cu_k[e], cu_k[e+1]);
  * a query row of document e sees only keys of document e, under the
    fixed-length rules (bottom-right causal alignment, window, GQA) applied to
    positions counted from the document's start;
  * decode with per-sequence lengths: sequence b's cache holds kv_lens[b]
    valid keys at the front of a [B, Hkv, Nk, d] buffer; its query sits at
    position kv_lens[b] - 1, and keys past kv_lens[b] do not exist for it.
    A sequence with no key gets O = 0, LSE = -inf.
  * paged KV cache ("Attention Research", section 2, which lists paged
    variants among attention kernel libraries; the KV cache itself is in
    "Quadratic Complexity Bottleneck"): pools of fixed-size pages
    [num_pages, Hkv, page_size, d] and a block table naming, for each
    sequence, the physical page of its j-th run of page_size keys.
"""

from __future__ import annotations

import numpy as np

from .attention import _f64, attention_ref, decode_ref, visible_mask, _head_rows


def _offsets(cu) -> np.ndarray:
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0 and be non-decreasing")
    return cu


def document_of(cu, idx) -> np.ndarray:
    """Document index of each packed row in ``idx`` (rows of empty documents never occur)."""
    cu = _offsets(cu)
    return np.searchsorted(cu, np.asarray(idx, dtype=np.int64), side="right") - 1


def packed_visible_mask(cu_q, cu_k, causal: bool, window: int, rows=None) -> np.ndarray:
    """Boolean [len(rows), total_k] over the whole packed sequence.

    Written as one mask over all packed rows and keys (block-diagonal by
    document), not per document: query row i may see key j iff both lie in
    the same document and the fixed-length rule holds for their in-document
    positions. Integer logic only.
    """
    cu_q, cu_k = _offsets(cu_q), _offsets(cu_k)
    if cu_q.size != cu_k.size:
        raise ValueError("cu_q and cu_k must describe the same documents")
    total_q, total_k = int(cu_q[-1]), int(cu_k[-1])
    i = np.arange(total_q, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(total_k, dtype=np.int64)
    di = document_of(cu_q, i)[:, None]
    dj = document_of(cu_k, j)[None, :]
    len_q = (cu_q[1:] - cu_q[:-1])[di]
    len_k = (cu_k[1:] - cu_k[:-1])[di]
    p = (i[:, None] - cu_q[di]) + (len_k - len_q)   # position within the document
    jl = j[None, :] - cu_k[dj]                       # key position within its document
    vis = di == dj
    if causal:
        vis &= jl <= p
    if window > 0:
        vis &= jl >= p - window
        if not causal:
            vis &= jl <= p + window
    return vis


def attention_varlen_ref(q, k, v, cu_q, cu_k, scale: float, causal: bool = False,
                         window: int = 0):
    """Packed attention: returns (O [H, total_q, d], LSE [H, total_q]) in float64.

    q [H, total_q, d], k/v [Hkv, total_k, d]. Because the mask is
    block-diagonal, each document is the fixed-length definition applied to
    its own rows and keys (B = 1).
    """
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    cu_q, cu_k = _offsets(cu_q), _offsets(cu_k)
    if cu_q.size != cu_k.size or cu_q[-1] != q64.shape[1] or cu_k[-1] != k64.shape[1]:
        raise ValueError("cu_seqlens do not match the packed tensors")
    H, total_q, _ = q64.shape
    o = np.zeros((H, total_q, v64.shape[2]))
    lse = np.full((H, total_q), -np.inf)
    for e in range(cu_q.size - 1):
        qs, qe, ks, ke = int(cu_q[e]), int(cu_q[e + 1]), int(cu_k[e]), int(cu_k[e + 1])
        if qe == qs:
            continue
        if ke == ks:  # no keys: every row of this document is empty
            continue
        od, ld = attention_ref(q64[None, :, qs:qe], k64[None, :, ks:ke], v64[None, :, ks:ke],
                               scale, causal, window)
        o[:, qs:qe] = od[0]
        lse[:, qs:qe] = ld[0]
    return o, lse


def attention_varlen_rows_ref(q, k, v, cu_q, cu_k, scale: float, causal: bool, window: int,
                              h: int, rows):
    """Selected packed query rows of head h: (O [r, d], LSE [r]) in float64."""
    cu_q, cu_k = _offsets(cu_q), _offsets(cu_k)
    H, Hkv = q.shape[0], k.shape[0]
    kvh = h // (H // Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    out_o = np.zeros((rows.size, v.shape[2]))
    out_l = np.full(rows.size, -np.inf)
    docs = document_of(cu_q, rows)
    for e in np.unique(docs):
        sel = np.nonzero(docs == e)[0]
        qs, ks, ke = int(cu_q[e]), int(cu_k[e]), int(cu_k[e + 1])
        len_q = int(cu_q[e + 1]) - qs
        if ke == ks:
            continue
        local = rows[sel] - qs
        vis = visible_mask(len_q, ke - ks, causal, window, local)
        qh = _f64(q[h][rows[sel]])
        kh, vh = _f64(k[kvh][ks:ke]), _f64(v[kvh][ks:ke])
        od, ld, _ = _head_rows(qh, kh, vh, float(scale), vis)
        out_o[sel] = od
        out_l[sel] = ld
    return out_o, out_l


def decode_kvlens_ref(q, k_cache, v_cache, kv_lens, scale: float, window: int = 0):
    """Decode with per-sequence cache lengths: (O [B,H,d], LSE [B,H]) in float64.

    Sequence b uses only the first kv_lens[b] rows of its cache; the query
    sits at the last of them.
    """
    q64 = _f64(q)
    B, H, d = q64.shape
    lens = np.asarray(kv_lens, dtype=np.int64)
    o = np.zeros((B, H, d))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        n = int(lens[b])
        if n <= 0:
            continue
        ob, lb = decode_ref(q64[b:b + 1], k_cache[b:b + 1, :, :n], v_cache[b:b + 1, :, :n],
                            scale, window)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse


def decode_kvlens_rows_ref(q, k_cache, v_cache, kv_lens, scale: float, window: int, b: int,
                           heads):
    """Decode output for chosen heads of sequence b (its cache read only up to kv_lens[b])."""
    n = int(kv_lens[b])
    H = q.shape[1]
    Hkv = k_cache.shape[1]
    G = H // Hkv
    if n <= 0:
        return np.zeros((len(heads), q.shape[2])), np.full(len(heads), -np.inf)
    q64 = _f64(q[b])
    vis = visible_mask(1, n, True, window)
    out_o, out_l, cache = [], [], {}
    for h in heads:
        kvh = h // G
        if kvh not in cache:
            cache[kvh] = (_f64(k_cache[b, kvh, :n]), _f64(v_cache[b, kvh, :n]))
        kh, vh = cache[kvh]
        od, ld, _ = _head_rows(q64[h:h + 1], kh, vh, float(scale), vis)
        out_o.append(od[0])
        out_l.append(ld[0])
    return np.stack(out_o), np.array(out_l)


def gather_pages(pages, block_table, b: int, n: int, page_size: int) -> np.ndarray:
    """Sequence b's first n cache rows [Hkv, n, d] from a page pool [P, Hkv, page_size, d].

    Key j of sequence b lives in physical page block_table[b][j // page_size],
    row j % page_size.
    """
    rows = []
    for j in range(0, n, page_size):
        pg = int(block_table[b][j // page_size])
        take = min(page_size, n - j)
        rows.append(_f64(pages[pg][:, :take]))
    if not rows:
        return np.zeros((pages.shape[1], 0, pages.shape[3]))
    return np.concatenate(rows, axis=1)


def decode_paged_ref(q, k_pages, v_pages, block_table, kv_lens, page_size: int, scale: float,
                     window: int = 0, seqs=None, heads=None):
    """Decode over a paged KV cache: (O [len(seqs), len(heads), d], LSE) in float64.

    Reading (the pages name paged KV caches without a layout): K and V pages
    form pools [num_pages, Hkv, page_size, d]; sequence b holds kv_lens[b]
    keys whose j-th page is block_table[b][j]. Each sequence is gathered into
    a contiguous cache and attended as in decode_kvlens_ref.
    """
    q64 = _f64(q)
    B, H, d = q64.shape
    Hkv = k_pages.shape[1]
    G = H // Hkv
    seqs = range(B) if seqs is None else list(seqs)
    heads = range(H) if heads is None else list(heads)
    o = np.zeros((len(seqs), len(heads), d))
    lse = np.full((len(seqs), len(heads)), -np.inf)
    for si, b in enumerate(seqs):
        n = int(kv_lens[b])
        if n <= 0:
            continue
        kb = gather_pages(k_pages, block_table, b, n, page_size)
        vb = gather_pages(v_pages, block_table, b, n, page_size)
        vis = visible_mask(1, n, True, window)
        for hi, h in enumerate(heads):
            od, ld, _ = _head_rows(q64[b, h:h + 1], kb[h // G], vb[h // G], float(scale), vis)
            o[si, hi], lse[si, hi] = od[0], ld[0]
    return o, lse
