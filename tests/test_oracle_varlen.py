"""Pins for the packed-sequence and per-sequence-length oracle (CPU only).

The pages fix one property of packing: the mask starts afresh at every
document boundary, so no token sees another document ("What Lost, and Why",
closing section). Each test checks the oracle against something other than
itself:

* brute force: scalar loops that find each row's document by a linear scan
  of the offsets and visit its keys as an explicit index range;
* no leakage: changing one document's K/V leaves every other document's
  output bit-identical;
* reduction: equal-length documents are the fixed-length batch (already
  pinned against torch and brute force), only laid out differently;
* decode: rows past a sequence's length never matter; a full-length
  sequence is plain decode; an empty one is O = 0, LSE = -inf;
* closed form: with q = 0 every visible score is 0, so LSE = ln(count);
* paged caches: scalar loops that address key j as (page j // page_size,
  row j % page_size); in-order pages equal the contiguous cache; moving pages
  physically (and the table with them) changes nothing; sequences naming the
  same physical pages share those keys.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import attention_ref, decode_ref
from oracle.varlen import document_of
from synth import inputs as S

RNG = np.random.default_rng(4321)


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def brute_packed(q, k, v, cu_q, cu_k, scale, causal, window):
    H, TQ, d = q.shape
    Hkv = k.shape[0]
    G = H // Hkv
    O = np.zeros((H, TQ, v.shape[2]))
    L = np.full((H, TQ), -math.inf)
    ndoc = len(cu_q) - 1
    for h in range(H):
        g = h // G
        for i in range(TQ):
            e = None
            for cand in range(ndoc):  # linear scan for the row's document
                if cu_q[cand] <= i < cu_q[cand + 1]:
                    e = cand
            lq, lk = cu_q[e + 1] - cu_q[e], cu_k[e + 1] - cu_k[e]
            pos = (i - cu_q[e]) + (lk - lq)
            first = max(0, pos - window) if window else 0
            if causal:
                last = min(pos, lk - 1)
            else:
                last = min(lk - 1, pos + window) if window else lk - 1
            keys = [int(cu_k[e]) + j for j in range(first, last + 1)]
            if not keys:
                continue
            sc = [scale * math.fsum(float(q[h, i, c]) * float(k[g, j, c]) for c in range(d))
                  for j in keys]
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            den = math.fsum(w)
            for c in range(v.shape[2]):
                O[h, i, c] = math.fsum(w[t] * float(v[g, keys[t], c]) for t in range(len(keys))) / den
            L[h, i] = mx + math.log(den)
    return O, L


# documents: (query lengths, key lengths); includes a document with keys but
# no queries, one with more queries than keys (leading rows empty under
# causal), and one with queries but no keys
DOCS = [
    ([3, 0, 5, 1, 4], [3, 2, 5, 1, 6]),
    ([2, 4, 3], [2, 2, 7]),
    ([3, 1], [0, 1]),
]


@pytest.mark.parametrize("docs", DOCS)
@pytest.mark.parametrize("causal,window", [(0, 0), (1, 0), (1, 1), (1, 3), (0, 2)])
@pytest.mark.parametrize("H,Hkv", [(4, 4), (4, 2), (2, 1)])
def test_varlen_brute_force(docs, causal, window, H, Hkv):
    lq, lk = docs
    cu_q, cu_k = _cu(lq), _cu(lk)
    d = 3
    q = RNG.standard_normal((H, cu_q[-1], d))
    k = RNG.standard_normal((Hkv, cu_k[-1], d))
    v = RNG.standard_normal((Hkv, cu_k[-1], 2))
    o, lse = oracle.attention_varlen_ref(q, k, v, cu_q, cu_k, 0.7, causal, window)
    bo, bl = brute_packed(q, k, v, cu_q, cu_k, 0.7, causal, window)
    assert np.array_equal(np.isinf(lse), np.isinf(bl))
    fin = np.isfinite(bl)
    assert np.max(np.abs(lse[fin] - bl[fin]), initial=0) < 1e-12
    assert np.max(np.abs(o - bo), initial=0) < 1e-12


@pytest.mark.parametrize("docs", DOCS)
@pytest.mark.parametrize("causal,window", [(0, 0), (1, 0), (1, 2), (0, 1)])
def test_packed_mask_brute_force(docs, causal, window):
    """The global block-diagonal mask, element by element."""
    lq, lk = docs
    cu_q, cu_k = _cu(lq), _cu(lk)
    vis = oracle.packed_visible_mask(cu_q, cu_k, causal, window)
    for i in range(cu_q[-1]):
        for j in range(cu_k[-1]):
            ei = [e for e in range(len(lq)) if cu_q[e] <= i < cu_q[e + 1]][0]
            ej = [e for e in range(len(lk)) if cu_k[e] <= j < cu_k[e + 1]][0]
            pos = i - cu_q[ei] + lk[ei] - lq[ei]
            jl = j - cu_k[ej]
            want = ei == ej
            if causal:
                want = want and jl <= pos
            if window:
                want = want and pos - window <= jl and (causal or jl <= pos + window)
            assert vis[i, j] == want, (i, j)


def test_document_of_skips_empty_documents():
    cu = _cu([2, 0, 0, 3, 1])
    assert list(document_of(cu, range(6))) == [0, 0, 3, 3, 3, 4]


@pytest.mark.parametrize("causal,window", [(1, 0), (0, 0), (1, 5)])
def test_no_leakage_between_documents(causal, window):
    lens = [7, 13, 1, 9]
    cu = _cu(lens)
    q = RNG.standard_normal((4, cu[-1], 8))
    k = RNG.standard_normal((2, cu[-1], 8))
    v = RNG.standard_normal((2, cu[-1], 8))
    o, lse = oracle.attention_varlen_ref(q, k, v, cu, cu, 0.5, causal, window)
    e = 1
    k2, v2 = k.copy(), v.copy()
    k2[:, cu[e]:cu[e + 1]] += 3.0
    v2[:, cu[e]:cu[e + 1]] -= 2.0
    o2, lse2 = oracle.attention_varlen_ref(q, k2, v2, cu, cu, 0.5, causal, window)
    inside = np.zeros(cu[-1], dtype=bool)
    inside[cu[e]:cu[e + 1]] = True
    assert np.array_equal(o[:, ~inside], o2[:, ~inside])
    assert np.array_equal(lse[:, ~inside], lse2[:, ~inside])
    assert np.all(np.abs(o[:, inside] - o2[:, inside]).max(axis=-1) > 1e-3)


@pytest.mark.parametrize("causal,window", [(1, 0), (0, 3), (1, 4)])
def test_equal_lengths_reduce_to_fixed_batch(causal, window):
    B, H, Hkv, N, d = 3, 4, 2, 11, 5
    q = RNG.standard_normal((B, H, N, d))
    k = RNG.standard_normal((B, Hkv, N, d))
    v = RNG.standard_normal((B, Hkv, N, d))
    ro, rl = attention_ref(q, k, v, 0.3, causal, window)
    pack = lambda x: np.ascontiguousarray(x.transpose(1, 0, 2, 3).reshape(x.shape[1], -1, d))
    cu = _cu([N] * B)
    o, lse = oracle.attention_varlen_ref(pack(q), pack(k), pack(v), cu, cu, 0.3, causal, window)
    assert np.max(np.abs(o - pack(ro))) < 1e-13
    assert np.max(np.abs(lse - rl.transpose(1, 0, 2).reshape(H, -1))) < 1e-13


def test_varlen_rows_match_full():
    lq, lk = [5, 9, 0, 4], [5, 12, 3, 2]
    cu_q, cu_k = _cu(lq), _cu(lk)
    q = RNG.standard_normal((4, cu_q[-1], 6))
    k = RNG.standard_normal((2, cu_k[-1], 6))
    v = RNG.standard_normal((2, cu_k[-1], 6))
    o, lse = oracle.attention_varlen_ref(q, k, v, cu_q, cu_k, 0.4, True, 3)
    rows = [0, 4, 5, 13, 14, 17]
    for h in range(4):
        ro, rl = oracle.attention_varlen_rows_ref(q, k, v, cu_q, cu_k, 0.4, True, 3, h, rows)
        assert np.max(np.abs(ro - o[h, rows])) < 1e-14
        assert np.array_equal(rl, lse[h, rows])


@pytest.mark.parametrize("causal,window", [(1, 0), (1, 6), (0, 0), (0, 4)])
def test_zero_queries_count_visible_keys(causal, window):
    lq, lk = [10, 3, 17, 1], [12, 3, 17, 5]
    cu_q, cu_k = _cu(lq), _cu(lk)
    q = np.zeros((2, cu_q[-1], 4))
    k = RNG.standard_normal((1, cu_k[-1], 4))
    v = RNG.standard_normal((1, cu_k[-1], 4))
    _, lse = oracle.attention_varlen_ref(q, k, v, cu_q, cu_k, 1.0, causal, window)
    for e in range(len(lq)):
        for r in range(lq[e]):
            pos = r + lk[e] - lq[e]
            if causal:
                n = min(pos, lk[e] - 1) + 1 - (max(0, pos - window) if window else 0)
            else:
                lo = max(0, pos - window) if window else 0
                hi = min(lk[e] - 1, pos + window) if window else lk[e] - 1
                n = hi - lo + 1
            want = math.log(n) if n > 0 else -math.inf
            assert lse[0, cu_q[e] + r] == pytest.approx(want, abs=1e-13)


# --------------------------------------------------------------------------
# decode with per-sequence cache lengths


def brute_decode(q, kc, vc, lens, scale, window):
    B, H, d = q.shape
    G = H // kc.shape[1]
    O = np.zeros((B, H, vc.shape[3]))
    L = np.full((B, H), -math.inf)
    for b in range(B):
        n = int(lens[b])
        for h in range(H):
            keys = list(range(max(0, n - 1 - window) if window else 0, n))
            if not keys:
                continue
            sc = [scale * math.fsum(q[b, h, c] * kc[b, h // G, j, c] for c in range(d)) for j in keys]
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            den = math.fsum(w)
            for c in range(vc.shape[3]):
                O[b, h, c] = math.fsum(w[t] * vc[b, h // G, keys[t], c] for t in range(len(keys))) / den
            L[b, h] = mx + math.log(den)
    return O, L


@pytest.mark.parametrize("window", [0, 2, 9])
def test_decode_kvlens_brute_force(window):
    B, H, Hkv, Nk, d = 5, 4, 2, 9, 3
    q = RNG.standard_normal((B, H, d))
    kc = RNG.standard_normal((B, Hkv, Nk, d))
    vc = RNG.standard_normal((B, Hkv, Nk, d))
    lens = np.array([9, 0, 1, 4, 7])
    o, lse = oracle.decode_kvlens_ref(q, kc, vc, lens, 0.6, window)
    bo, bl = brute_decode(q, kc, vc, lens, 0.6, window)
    assert np.array_equal(np.isinf(lse), np.isinf(bl))
    fin = np.isfinite(bl)
    assert np.max(np.abs(lse[fin] - bl[fin])) < 1e-12
    assert np.max(np.abs(o - bo)) < 1e-12
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))


def test_decode_kvlens_ignores_rows_past_length():
    B, H, Hkv, Nk, d = 4, 4, 1, 16, 4
    q = RNG.standard_normal((B, H, d))
    kc = RNG.standard_normal((B, Hkv, Nk, d))
    vc = RNG.standard_normal((B, Hkv, Nk, d))
    lens = np.array([16, 3, 11, 1])
    o, lse = oracle.decode_kvlens_ref(q, kc, vc, lens, 0.5, 0)
    kc2, vc2 = kc.copy(), vc.copy()
    for b in range(B):
        kc2[b, :, lens[b]:] = 1e3
        vc2[b, :, lens[b]:] = -1e3
    o2, lse2 = oracle.decode_kvlens_ref(q, kc2, vc2, lens, 0.5, 0)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    full_o, full_l = decode_ref(q[:1], kc[:1], vc[:1], 0.5, 0)
    assert np.max(np.abs(o[0] - full_o[0])) < 1e-15


def test_decode_kvlens_rows_match_full():
    B, H, Hkv, Nk, d = 3, 8, 2, 20, 4
    q = RNG.standard_normal((B, H, d))
    kc = RNG.standard_normal((B, Hkv, Nk, d))
    vc = RNG.standard_normal((B, Hkv, Nk, d))
    lens = np.array([20, 0, 13])
    o, lse = oracle.decode_kvlens_ref(q, kc, vc, lens, 0.5, 5)
    for b in range(B):
        ro, rl = oracle.decode_kvlens_rows_ref(q, kc, vc, lens, 0.5, 5, b, [0, 3, 7])
        assert np.max(np.abs(ro - o[b, [0, 3, 7]])) < 1e-14
        assert np.array_equal(rl, lse[b, [0, 3, 7]])


# --------------------------------------------------------------------------
# the seeded length generators


def test_packed_lengths_fill_contexts():
    cfg = S.PACKED["packed_24docs_4x8192_d128"]
    lens = cfg.lengths(0)
    assert sum(lens) == cfg.contexts * cfg.context_len
    assert all(1 <= n <= cfg.max_len for n in lens)
    # documents never span contexts: the running totals hit every boundary
    ends = set(np.cumsum(lens).tolist())
    for c in range(1, cfg.contexts + 1):
        assert c * cfg.context_len in ends
    assert lens == cfg.lengths(0) and lens != cfg.lengths(1)
    cu = S.cu_seqlens(lens)
    assert cu.dtype == np.int32 and cu[0] == 0 and cu[-1] == sum(lens)


def test_kv_lengths_range():
    lens = S.kv_lengths(0, 64, 32768)
    assert lens.dtype == np.int32 and lens.min() >= 1 and lens.max() <= 32768
    assert np.array_equal(lens, S.kv_lengths(0, 64, 32768))


# --------------------------------------------------------------------------
# decode over a paged cache


def brute_paged(q, kp, vp, table, lens, ps, scale, window):
    B, H, d = q.shape
    G = H // kp.shape[1]
    O = np.zeros((B, H, vp.shape[3]))
    L = np.full((B, H), -math.inf)
    for b in range(B):
        n = int(lens[b])
        keys = list(range(max(0, n - 1 - window) if window else 0, n))
        for h in range(H):
            if not keys:
                continue
            g = h // G
            addr = [(int(table[b][j // ps]), j % ps) for j in keys]
            sc = [scale * math.fsum(q[b, h, c] * kp[pg, g, r, c] for c in range(d)) for pg, r in addr]
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            den = math.fsum(w)
            for c in range(vp.shape[3]):
                O[b, h, c] = math.fsum(w[t] * vp[pg, g, r, c] for t, (pg, r) in enumerate(addr)) / den
            L[b, h] = mx + math.log(den)
    return O, L


@pytest.mark.parametrize("ps", [2, 4])
@pytest.mark.parametrize("window", [0, 3])
def test_paged_brute_force(ps, window):
    lens = np.array([7, 0, 1, 8, 5])
    table, npg = S.paged_block_table(3, lens, ps)
    H, Hkv, d = 4, 2, 3
    q = RNG.standard_normal((len(lens), H, d))
    kp = RNG.standard_normal((npg, Hkv, ps, d))
    vp = RNG.standard_normal((npg, Hkv, ps, d))
    o, lse = oracle.decode_paged_ref(q, kp, vp, table, lens, ps, 0.7, window)
    bo, bl = brute_paged(q, kp, vp, table, lens, ps, 0.7, window)
    assert np.array_equal(np.isinf(lse), np.isinf(bl))
    fin = np.isfinite(bl)
    assert np.max(np.abs(lse[fin] - bl[fin])) < 1e-12
    assert np.max(np.abs(o - bo)) < 1e-12


def test_paged_in_order_pages_equal_contiguous_cache():
    B, H, Hkv, Nk, d, ps = 3, 4, 2, 12, 5, 4
    q = RNG.standard_normal((B, H, d))
    kc = RNG.standard_normal((B, Hkv, Nk, d))
    vc = RNG.standard_normal((B, Hkv, Nk, d))
    lens = np.array([12, 5, 9])
    mp = Nk // ps
    to_pages = lambda c: c.reshape(B, Hkv, mp, ps, d).transpose(0, 2, 1, 3, 4).reshape(B * mp, Hkv, ps, d)
    table = np.arange(B * mp).reshape(B, mp)
    o, lse = oracle.decode_paged_ref(q, to_pages(kc), to_pages(vc), table, lens, ps, 0.4, 0)
    ro, rl = oracle.decode_kvlens_ref(q, kc, vc, lens, 0.4, 0)
    assert np.max(np.abs(o - ro)) < 1e-14 and np.max(np.abs(lse - rl)) < 1e-14


def test_paged_physical_permutation_is_invisible():
    lens = np.array([9, 14, 3])
    ps = 4
    table, npg = S.paged_block_table(0, lens, ps)
    q = RNG.standard_normal((3, 4, 6))
    kp = RNG.standard_normal((npg, 1, ps, 6))
    vp = RNG.standard_normal((npg, 1, ps, 6))
    o, lse = oracle.decode_paged_ref(q, kp, vp, table, lens, ps, 0.5, 0)
    perm = RNG.permutation(npg)          # physical page p moves to slot perm[p]
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1)
    o2, lse2 = oracle.decode_paged_ref(q, kp2, vp2, table2, lens, ps, 0.5, 0)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_paged_shared_prefix_pages():
    """Two sequences naming the same physical pages see the same keys."""
    ps = 4
    kp = RNG.standard_normal((5, 1, ps, 3))
    vp = RNG.standard_normal((5, 1, ps, 3))
    q = np.repeat(RNG.standard_normal((1, 2, 3)), 2, axis=0)
    table = np.array([[0, 1, 2], [0, 1, 4]])
    o, lse = oracle.decode_paged_ref(q, kp, vp, table, [10, 8], ps, 0.5, 0)
    ro, rl = oracle.decode_paged_ref(q[:1], kp, vp, table[:1], [8], ps, 0.5, 0)
    assert np.array_equal(o[1], ro[0]) and np.array_equal(lse[1], rl[0])


def test_paged_block_table_generator():
    lens = S.kv_lengths(0, 64, 32768)
    table, npg = S.paged_block_table(0, lens, 16)
    need = -(-lens.astype(np.int64) // 16)
    assert npg == need.sum() and table.shape == (64, need.max())
    used = np.concatenate([table[b, :need[b]] for b in range(64)])
    assert np.array_equal(np.sort(used), np.arange(npg))          # each page once
    assert all(np.all(table[b, need[b]:] == -1) for b in range(64))
