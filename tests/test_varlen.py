"""Packed documents and per-sequence cache lengths: HIP path against the oracle.

Prefill (attn_fwd_varlen): element-wise parity on small packed batches that
span several tiles with ragged tails, empty documents, documents with more
or fewer queries than keys, and documents with no keys; exact mask checks
(q = 0 counts, bit-identical output of the other documents when one is
changed); per-document tile counts; equal-length documents equal the
fixed-length kernel bit for bit. (The packed workload at full size is
compared on every output in test_full_size.py.)

Decode (attn_decode_varlen): parity on mixed lengths including 0 and 1;
work-group runs of tiles that cross sequences, or find none; cache rows past
a sequence's length never matter; full-length sequences equal attn_decode
bit for bit where its equal chunks are whole tiles; each sequence equals a one-query packed
prefill over its keys. (The mixed-length workload at full size is compared on
every output in test_full_size.py.)
"""

import math

import numpy as np
import pytest
import torch

import oracle
import exact_io_aware_06_amd as mi
from helpers import check_lse, check_out, to64
from synth import inputs as S

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _gen(seed):
    return torch.Generator(device="cpu").manual_seed(seed)


def packed_case(lq, lk, H, Hkv, d, seed):
    g = _gen(seed)
    q = torch.randn(H, sum(lq), d, generator=g).to(torch.bfloat16)
    k = torch.randn(Hkv, sum(lk), d, generator=g).to(torch.bfloat16)
    v = torch.randn(Hkv, sum(lk), d, generator=g).to(torch.bfloat16)
    return q, k, v, S.cu_seqlens(lq), S.cu_seqlens(lk)


def run_varlen(q, k, v, cu_q, cu_k, scale, causal, window, max_q=None):
    lq = np.diff(cu_q)
    max_q = int(lq.max(initial=0)) if max_q is None else max_q
    o, lse = mi.attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV),
                                torch.from_numpy(cu_q).to(DEV), torch.from_numpy(cu_k).to(DEV),
                                max_q, scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    return o, lse


DOC_CASES = [
    # (query lengths, key lengths): self-attention mixes with ragged tails
    ([300, 1, 129, 64, 700], [300, 1, 129, 64, 700]),
    ([1000, 0, 77, 256], [1000, 0, 77, 256]),
    # more keys than queries (a cached prefix), fewer keys than queries
    # (leading rows empty under causal), a document with queries but no keys
    ([100, 200, 50, 33], [400, 150, 0, 33]),
    ([5, 130, 1], [260, 3, 1]),
]


@pytest.mark.parametrize("docs", DOC_CASES)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,window", [(1, 0), (0, 0), (1, 100), (0, 64)])
def test_varlen_parity(docs, d, causal, window):
    lq, lk = docs
    H, Hkv = 8, 2
    q, k, v, cu_q, cu_k = packed_case(lq, lk, H, Hkv, d, seed=len(lq) * 10 + d + causal)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = run_varlen(q, k, v, cu_q, cu_k, scale, causal, window)
    o_ref, l_ref = oracle.attention_varlen_ref(q, k, v, cu_q, cu_k, scale, causal, window)
    label = f"docs={lq}/{lk} d={d} causal={causal} W={window}"
    check_out(to64(o), o_ref, bf16=True, label=label)
    check_lse(to64(lse), l_ref, label=label)


@pytest.mark.parametrize("docs", DOC_CASES)
@pytest.mark.parametrize("causal,window", [(1, 0), (1, 37), (0, 0), (0, 5)])
def test_varlen_zero_queries_count_visible_keys(docs, causal, window):
    """q = 0: every visible score is 0, so exp(LSE) is the exact visible count."""
    lq, lk = docs
    q, k, v, cu_q, cu_k = packed_case(lq, lk, 4, 1, 128, seed=3)
    q.zero_()
    _, lse = run_varlen(q, k, v, cu_q, cu_k, 1.0, causal, window)
    count = oracle.packed_visible_mask(cu_q, cu_k, causal, window).sum(axis=1)
    lg = to64(lse)
    for h in range(4):
        got = np.where(np.isneginf(lg[h]), 0, np.rint(np.exp(lg[h])))
        assert np.array_equal(got.astype(np.int64), count), f"head {h}"


@pytest.mark.parametrize("causal,window", [(1, 0), (0, 0), (1, 50)])
def test_varlen_no_leakage(causal, window):
    """Changing one document's K/V leaves every other row bit-identical."""
    lq = [200, 129, 64, 300]
    q, k, v, cu_q, cu_k = packed_case(lq, lq, 8, 2, 128, seed=11)
    o1, l1 = run_varlen(q, k, v, cu_q, cu_k, 0.088, causal, window)
    e = 1
    k2, v2 = k.clone(), v.clone()
    k2[:, cu_k[e]:cu_k[e + 1]] = torch.randn(2, lq[e], 128, generator=_gen(99)).to(torch.bfloat16)
    v2[:, cu_k[e]:cu_k[e + 1]] = 5.0
    o2, l2 = run_varlen(q, k2, v2, cu_q, cu_k, 0.088, causal, window)
    inside = torch.zeros(sum(lq), dtype=torch.bool, device=DEV)
    inside[cu_q[e]:cu_q[e + 1]] = True
    assert torch.equal(o1[:, ~inside], o2[:, ~inside])
    assert torch.equal(l1[:, ~inside], l2[:, ~inside])
    assert not torch.equal(o1[:, inside], o2[:, inside])


@pytest.mark.parametrize("causal,window", [(1, 0), (0, 0), (1, 300)])
def test_varlen_equal_lengths_match_fixed_kernel(causal, window):
    """Documents of equal length N are the fixed-length batch, bit for bit."""
    B, H, Hkv, N, d = 3, 8, 2, 640, 128
    g = _gen(21)
    q = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16).to(DEV)
    o_fix, l_fix = mi.attn_fwd(q, k, v, scale=0.088, causal=causal, window=window)
    pack = lambda x: x.transpose(0, 1).reshape(x.shape[1], B * N, d).contiguous()
    cu = S.cu_seqlens([N] * B)
    o, lse = run_varlen(pack(q), pack(k), pack(v), cu, cu, 0.088, causal, window)
    assert torch.equal(o, pack(o_fix))
    assert torch.equal(lse, l_fix.transpose(0, 1).reshape(H, B * N))


@pytest.mark.parametrize("docs", DOC_CASES)
@pytest.mark.parametrize("causal,window", [(1, 0), (0, 0), (1, 100), (0, 64)])
def test_varlen_only_visible_tiles_are_loaded(docs, causal, window):
    """Per document, exactly the blocks holding a visible pair are loaded;
    work-groups past a document's end load nothing."""
    lq, lk = docs
    H, d = 4, 128
    q, k, v, cu_q, cu_k = packed_case(lq, lk, H, 2, d, seed=5)
    max_q = max(lq)
    o, lse, counts = mi.fwd_varlen_tile_counts(
        q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(cu_q).to(DEV),
        torch.from_numpy(cu_k).to(DEV), max_q, scale=0.1, causal=causal, window=window)
    o2, l2 = run_varlen(q, k, v, cu_q, cu_k, 0.1, causal, window)
    assert torch.equal(o, o2) and torch.equal(lse, l2)  # instrumentation changes nothing
    bm, bn = mi.fwd_tile_shape(d)
    counts = counts.cpu().numpy()
    nqt = -(-max_q // bm)
    for e, (nq, nk) in enumerate(zip(lq, lk)):
        loaded = np.zeros(nqt, dtype=np.int64)
        masked = np.zeros(nqt, dtype=np.int64)
        if nq > 0 and nk > 0:
            need, full = oracle.tiles_needed(nq, nk, causal, window, bm, bn)
            loaded[:need.shape[0]] = need.sum(axis=1)
            masked[:need.shape[0]] = (need & ~full).sum(axis=1)
        for h in range(H):
            assert np.array_equal(counts[e, h, :, 0], loaded), f"doc {e} head {h}"
            assert np.array_equal(counts[e, h, :, 1], masked), f"doc {e} head {h}"


def test_varlen_bad_offsets_skip_the_document():
    """Offsets past the packed tensors: that document is skipped, others are right."""
    lq = [100, 60, 40]
    q, k, v, cu_q, cu_k = packed_case(lq, lq, 4, 2, 64, seed=8)
    bad_q, bad_k = cu_q.copy(), cu_k.copy()
    bad_q[2], bad_k[2] = 10_000, 10_000       # doc 1 ends past the end, doc 2 starts there
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o = torch.full_like(qd, 7.0)
    lse = torch.full((4, sum(lq)), 7.0, device=DEV)
    mi.attn_fwd_varlen(qd, kd, vd, torch.from_numpy(bad_q).to(DEV),
                       torch.from_numpy(bad_k).to(DEV), 100, scale=0.125, causal=True,
                       out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen_ref(q, k, v, cu_q, cu_k, 0.125, True, 0)
    check_out(to64(o[:, :100]), o_ref[:, :100], label="doc 0")
    check_lse(to64(lse[:, :100]), l_ref[:, :100], label="doc 0")
    assert torch.all(o[:, 100:] == 7.0) and torch.all(lse[:, 100:] == 7.0)


def test_varlen_rows_past_max_seqlen_are_not_written():
    lq = [300, 100]
    q, k, v, cu_q, cu_k = packed_case(lq, lq, 2, 1, 128, seed=9)
    qd = q.to(DEV)
    o = torch.full_like(qd, 3.0)
    lse = torch.full((2, 400), 3.0, device=DEV)
    mi.attn_fwd_varlen(qd, k.to(DEV), v.to(DEV), torch.from_numpy(cu_q).to(DEV),
                       torch.from_numpy(cu_k).to(DEV), 128, scale=0.09, causal=True,
                       out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen_ref(q, k, v, cu_q, cu_k, 0.09, True, 0)
    written = np.r_[0:128, 300:400]
    check_out(to64(o[:, written]), o_ref[:, written], label="written rows")
    assert torch.all(o[:, 128:300] == 3.0) and torch.all(lse[:, 128:300] == 3.0)


# --------------------------------------------------------------------------
# decode with per-sequence cache lengths


def run_decode(q, kc, vc, lens, scale, window, splits):
    o, lse = mi.attn_decode_varlen(q.to(DEV), kc.to(DEV), vc.to(DEV),
                                   torch.as_tensor(lens, dtype=torch.int32).to(DEV),
                                   scale=scale, window=window, num_splits=splits)
    torch.cuda.synchronize()
    return o, lse


def decode_case(B, H, Hkv, Nk, d, seed):
    g = _gen(seed)
    q = torch.randn(B, H, d, generator=g).to(torch.bfloat16)
    kc = torch.randn(B, Hkv, Nk, d, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Hkv, Nk, d, generator=g).to(torch.bfloat16)
    return q, kc, vc


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits,window", [(1, 0), (3, 0), (16, 0), (0, 0), (7, 40)])
def test_decode_varlen_parity(d, splits, window):
    lens = [0, 1, 17, 128, 129, 500, 1000]
    q, kc, vc = decode_case(len(lens), 8, 2, 1000, d, seed=d + splits)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = run_decode(q, kc, vc, lens, scale, window, splits)
    o_ref, l_ref = oracle.decode_kvlens_ref(q, kc, vc, lens, scale, window)
    label = f"d={d} splits={splits} W={window}"
    check_out(to64(o), o_ref, label=label)
    check_lse(to64(lse), l_ref, label=label)
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits,window", [(1, 0), (2, 0), (16, 0), (3, 50)])
def test_decode_varlen_pieces_span_sequences(d, splits, window):
    """Many short and empty sequences (23 key tiles in all, 16 sequences): with one split a
    work-group's run of tiles crosses several sequences; with 16 splits most of the 256
    work-groups per KV head get no tile at all."""
    lens = [0, 1, 5, 127, 128, 129, 0, 300, 2, 64, 1000, 0, 3, 256, 17, 0]
    q, kc, vc = decode_case(len(lens), 8, 2, 1000, d, seed=11 + d)
    o, lse = run_decode(q, kc, vc, lens, 0.088, window, splits)
    o_ref, l_ref = oracle.decode_kvlens_ref(q, kc, vc, lens, 0.088, window)
    label = f"d={d} splits={splits} W={window}"
    check_out(to64(o), o_ref, label=label)
    check_lse(to64(lse), l_ref, label=label)
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.all(o[b] == 0) and torch.all(torch.isneginf(lse[b]))


def test_decode_varlen_large_batch():
    """300 sequences: the plan's running sum over the batch takes two rounds of its 256
    threads."""
    rng = np.random.default_rng(13)
    lens = rng.integers(0, 301, size=300).tolist()
    lens[:3] = [0, 300, 1]
    q, kc, vc = decode_case(len(lens), 4, 1, 300, 64, seed=13)
    o, lse = run_decode(q, kc, vc, lens, 0.125, 0, 2)
    o_ref, l_ref = oracle.decode_kvlens_ref(q, kc, vc, lens, 0.125, 0)
    check_out(to64(o), o_ref, label="B=300")
    check_lse(to64(lse), l_ref, label="B=300")


def test_decode_varlen_skewed_batch():
    """One long sequence among one-key ones (157 + 31 tiles for up to 512 work-groups per KV
    head): each work-group takes one tile, so the long sequence's keys come back as 157
    partials, which the merge combines over three rounds of its 64 lanes."""
    lens = [20000] + [1] * 31
    q, kc, vc = decode_case(len(lens), 8, 2, 20000, 128, seed=12)
    o, lse = run_decode(q, kc, vc, lens, 0.088, 0, 16)
    o_ref, l_ref = oracle.decode_kvlens_ref(q, kc, vc, lens, 0.088, 0)
    check_out(to64(o), o_ref, label="skewed")
    check_lse(to64(lse), l_ref, label="skewed")


@pytest.mark.parametrize("H,Hkv", [(40, 1), (64, 1)])
def test_decode_varlen_many_heads_per_group(H, Hkv):
    lens = [0, 1, 200, 333]
    q, kc, vc = decode_case(len(lens), H, Hkv, 333, 128, seed=H)
    o, lse = run_decode(q, kc, vc, lens, 0.088, 0, 5)
    o_ref, l_ref = oracle.decode_kvlens_ref(q, kc, vc, lens, 0.088, 0)
    check_out(to64(o), o_ref, label=f"H={H}")
    check_lse(to64(lse), l_ref, label=f"H={H}")


def test_decode_varlen_ignores_rows_past_length():
    lens = [3, 700, 1000, 64]
    q, kc, vc = decode_case(4, 8, 2, 1000, 128, seed=2)
    o1, l1 = run_decode(q, kc, vc, lens, 0.088, 0, 8)
    kc2, vc2 = kc.clone(), vc.clone()
    for b, n in enumerate(lens):
        kc2[b, :, n:] = 300.0
        vc2[b, :, n:] = -300.0
    o2, l2 = run_decode(q, kc2, vc2, lens, 0.088, 0, 8)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("Nk,splits", [(777, 1), (4000, 1), (1280, 5), (2048, 16), (4096, 8)])
def test_decode_varlen_full_lengths_match_uniform_kernel(Nk, splits):
    """All lengths equal to Nk. With one chunk per sequence the balanced plan gives each
    work-group one whole sequence (its virtual tile and all its keys), the uniform kernel's
    chunk, so the two agree bit for bit. With S chunks the plan's runs are shifted by one
    virtual tile per sequence against the equal chunks: the same keys in other pieces. The
    merge combines any partition exactly in exact arithmetic, but each piece rounds P to bf16
    relative to its own reference maximum, which depends on where the piece starts, so here
    both results are held to the oracle's bound instead of to each other."""
    q, kc, vc = decode_case(3, 32, 8, Nk, 128, seed=4)
    o1, l1 = run_decode(q, kc, vc, [Nk] * 3, 0.088, 0, splits)
    o2, l2 = mi.attn_decode(q.to(DEV), kc.to(DEV), vc.to(DEV), scale=0.088, num_splits=splits)
    torch.cuda.synchronize()
    if splits == 1:
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        return
    o_ref, l_ref = oracle.decode_kvlens_ref(q, kc, vc, [Nk] * 3, 0.088, 0)
    for o, lse, name in ((o1, l1, "per-sequence lengths"), (o2, l2, "equal chunks")):
        check_out(to64(o), o_ref, label=f"{name} Nk={Nk} S={splits}")
        check_lse(to64(lse), l_ref, label=f"{name} Nk={Nk} S={splits}")


@pytest.mark.parametrize("B", [256, 257, 300])
def test_decode_varlen_large_batches(B):
    """Up to 256 sequences every split work-group plans its own run of tiles; past that a
    separate plan kernel writes the plan first. Both sides of the boundary, with empty,
    one-key and ragged sequences, against the oracle."""
    r = np.random.default_rng(B)
    lens = [int(x) for x in r.choice([0, 1, 64, 129, int(r.integers(0, 300))], B)]
    lens[-1] = 300  # a full sequence at the end of the batch
    q, kc, vc = decode_case(B, 4, 2, 300, 64, seed=B)
    o, lse = run_decode(q, kc, vc, lens, 0.125, 0, 3)
    o_ref, l_ref = oracle.decode_kvlens_ref(q, kc, vc, lens, 0.125, 0)
    check_out(to64(o), o_ref, label=f"B={B}")
    check_lse(to64(lse), l_ref, label=f"B={B}")
    empty = [b for b, n in enumerate(lens) if n == 0]
    assert torch.all(o[empty] == 0) and torch.all(torch.isneginf(lse[empty]))


def test_decode_varlen_matches_one_query_packed_prefill():
    """Sequence b is a one-query document over its kv_lens[b] keys."""
    lens = [1, 90, 300, 129]
    B, H, Hkv, Nk, d = len(lens), 8, 2, 300, 128
    q, kc, vc = decode_case(B, H, Hkv, Nk, d, seed=6)
    o_dec, l_dec = run_decode(q, kc, vc, lens, 0.088, 0, 4)
    qp = q.transpose(0, 1).contiguous()                      # [H, B, d]: one row per document
    kp = torch.cat([kc[b, :, :n] for b, n in enumerate(lens)], dim=1).contiguous()
    vp = torch.cat([vc[b, :, :n] for b, n in enumerate(lens)], dim=1).contiguous()
    o_pre, l_pre = run_varlen(qp, kp, vp, S.cu_seqlens([1] * B), S.cu_seqlens(lens), 0.088,
                              True, 0)
    ref_o, ref_l = oracle.decode_kvlens_ref(q, kc, vc, lens, 0.088, 0)
    check_out(to64(o_dec), ref_o, label="decode")
    check_out(to64(o_pre.transpose(0, 1)), ref_o, label="packed prefill")
    assert float((o_dec.float() - o_pre.transpose(0, 1).float()).abs().max()) <= 2e-2
    check_lse(to64(l_pre.transpose(0, 1)), ref_l, label="packed prefill lse")
