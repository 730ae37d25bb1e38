"""Bit-exact checks of the mask and tile indexing of the bf16 forward kernel.

* q = 0 makes every visible score 0, so LSE_i = ln |visible keys of row i|
  exactly enough that round(exp(LSE_i)) recovers the integer count.
* q = 0 and V[j, c] = [c == j mod d] give O_i[c] * |vis_i| = the number of
  visible keys of row i congruent to c mod d: the visible SET, not just its size.
* The instrumented launch reports, per work-group, the key tiles it loaded and
  how many of those it masked; they must equal the blocks of the score matrix
  that hold any visible pair (and those that hold a hidden one), computed by
  brute force from the visibility definition.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import visible_mask
import exact_io_aware_06_amd as mi

pytestmark = pytest.mark.gpu

DEV = "cuda"

SHAPES = [
    # B, H, Hkv, Nq, Nk, d, causal, window
    (4, 2, 2, 2048, 2048, 64, 1, 0),       # causal d=64 (2k context)
    (1, 4, 1, 8192, 8192, 128, 1, 0),      # causal GQA d=128 (8k)
    (1, 2, 1, 32768, 32768, 128, 1, 4096),  # causal window 4096 at 32k
    (1, 2, 1, 1000, 1300, 128, 1, 77),     # ragged, Nq < Nk
    (1, 2, 1, 1300, 1000, 64, 1, 0),       # Nq > Nk: empty rows
    (1, 2, 2, 777, 777, 128, 0, 100),      # two-sided window
    (1, 2, 2, 300, 300, 64, 0, 0),
    (1, 2, 1, 500, 500, 128, 1, 5000),     # window wider than the keys
    (1, 2, 1, 640, 640, 128, 1, 64),       # window on a key-tile boundary
    (1, 2, 1, 700, 900, 64, 1, 1),         # window of one key
    (1, 2, 2, 640, 640, 128, 0, 65),       # two-sided, one past a tile boundary
    (1, 2, 1, 1, 1000, 128, 1, 0),         # a single query row
    (1, 2, 1, 200, 4000, 128, 0, 5000),    # two-sided window wider than the keys
]


def row_counts(Nq, Nk, causal, window):
    out = np.empty(Nq, dtype=np.int64)
    for r0 in range(0, Nq, 2048):
        rows = np.arange(r0, min(Nq, r0 + 2048))
        out[rows] = visible_mask(Nq, Nk, causal, window, rows).sum(axis=1)
    return out


def inputs(B, H, Hkv, Nq, Nk, d, onehot_v):
    q = torch.zeros(B, H, Nq, d, dtype=torch.bfloat16, device=DEV)
    k = torch.ones(B, Hkv, Nk, d, dtype=torch.bfloat16, device=DEV)
    if onehot_v:
        j = torch.arange(Nk, device=DEV)
        v = torch.zeros(B, Hkv, Nk, d, dtype=torch.bfloat16, device=DEV)
        v[:, :, j, j % d] = 1
    else:
        v = torch.ones(B, Hkv, Nk, d, dtype=torch.bfloat16, device=DEV)
    return q, k, v


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,window", SHAPES)
def test_zero_queries_count_visible_keys(B, H, Hkv, Nq, Nk, d, causal, window):
    q, k, v = inputs(B, H, Hkv, Nq, Nk, d, onehot_v=False)
    o, lse = mi.attn_fwd(q, k, v, scale=0.125, causal=causal, window=window)
    torch.cuda.synchronize()
    cnt = row_counts(Nq, Nk, causal, window)
    lse = lse.double().cpu().numpy()
    for b in range(B):
        for h in range(H):
            l = lse[b, h]
            empty = cnt == 0
            assert np.all(np.isneginf(l[empty]))
            got = np.rint(np.exp(l[~empty])).astype(np.int64)
            bad = np.nonzero(got != cnt[~empty])[0]
            assert bad.size == 0, f"rows {bad[:5]} count {got[bad[:5]]} vs {cnt[~empty][bad[:5]]}"
    # V = 1 gives exactly 1 on every row that sees a key
    o = o.float().cpu().numpy()
    assert np.all(o[:, :, cnt > 0] == 1.0)
    assert np.all(o[:, :, cnt == 0] == 0.0)


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,window", SHAPES)
def test_zero_queries_recover_visible_set_mod_d(B, H, Hkv, Nq, Nk, d, causal, window):
    q, k, v = inputs(1, 1, 1, Nq, Nk, d, onehot_v=True)
    o, _ = mi.attn_fwd(q, k, v, scale=0.125, causal=causal, window=window)
    torch.cuda.synchronize()
    o = o.double().cpu().numpy()[0, 0]
    for r0 in range(0, Nq, 2048):
        rows = np.arange(r0, min(Nq, r0 + 2048))
        vis = visible_mask(Nq, Nk, causal, window, rows)
        cnt = vis.sum(axis=1)
        per_class = np.zeros((rows.size, d), dtype=np.int64)
        for c in range(d):
            per_class[:, c] = vis[:, c::d].sum(axis=1)
        assert per_class.max() <= 256  # bf16 keeps n / |vis| exact enough below this
        got = np.rint(o[rows] * cnt[:, None]).astype(np.int64)
        assert np.array_equal(got, per_class)


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,window", SHAPES)
def test_only_visible_tiles_are_loaded(B, H, Hkv, Nq, Nk, d, causal, window):
    gen = torch.Generator(device=DEV).manual_seed(5)
    q = torch.randn(B, H, Nq, d, device=DEV, generator=gen).to(torch.bfloat16)
    k = torch.randn(B, Hkv, Nk, d, device=DEV, generator=gen).to(torch.bfloat16)
    v = torch.randn(B, Hkv, Nk, d, device=DEV, generator=gen).to(torch.bfloat16)
    o, lse, counts = mi.fwd_tile_counts(q, k, v, scale=0.125, causal=causal, window=window)
    o2, lse2 = mi.attn_fwd(q, k, v, scale=0.125, causal=causal, window=window)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)  # instrumentation changes nothing
    bm, bn = mi.fwd_tile_shape(d)
    need, full = oracle.tiles_needed(Nq, Nk, causal, window, bm, bn)
    counts = counts.cpu().numpy()
    want_loaded = need.sum(axis=1)
    want_masked = (need & ~full).sum(axis=1)
    for b in range(B):
        for h in range(H):
            assert np.array_equal(counts[b, h, :, 0], want_loaded)
            assert np.array_equal(counts[b, h, :, 1], want_masked)
