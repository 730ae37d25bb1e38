"""Seeded random-shape parity sweeps of the forward, the backward and decode.

The fixed case lists elsewhere pick shapes by hand; these draw them: query
and key counts from 1 to 700 (Nq > Nk, Nq < Nk and ragged tails of every
tile size), d in {64, 128}, group sizes 1 to 8, causal or not, no window or
a window from 1 to 300 keys, and plain or sharpened logits (which drive the
online softmax's reference maximum to move often). Every draw is a fixed
function of its index, so a failure names a reproducible case. Forward
outputs are held to the forward tolerances of helpers.py; gradients to the
derived element-wise bound of test_bwd.py. The decode sweep draws batches of
per-sequence cache lengths (some empty), group sizes up to 40, split counts
and page sizes, and runs each case on contiguous caches, with the lengths,
and from a shuffled page pool. The packed sweep draws document counts and
lengths (documents without queries or keys included) for the packed forward
and backward.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from helpers import check_lse, check_out, to64
import exact_io_aware_06_amd as mi
from test_bwd import check as check_bwd

pytestmark = pytest.mark.gpu

DEV = "cuda"


def draw(i: int):
    """Shape, flags and inputs of random case i."""
    r = np.random.default_rng(1000 + i)
    d = int(r.choice([64, 128]))
    G = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.integers(1, 3))
    B = int(r.integers(1, 3))
    Nq = int(r.integers(1, 701))
    Nk = int(r.integers(1, 701)) if r.random() < 0.5 else Nq
    causal = int(r.random() < 0.6)
    window = 0 if r.random() < 0.5 else int(r.integers(1, 301))
    sharp = r.random() < 0.3
    mult = 3.0 * d ** -0.25 if sharp else 1.0
    scale = 1.0 if sharp else float(np.float32(1 / math.sqrt(d)))
    g = torch.Generator().manual_seed(7000 + i)
    H = Hkv * G
    f = lambda *s: (torch.randn(*s, generator=g) * mult).to(torch.bfloat16)
    q, k = f(B, H, Nq, d), f(B, Hkv, Nk, d)
    v = torch.randn(B, Hkv, Nk, d, generator=g).to(torch.bfloat16)
    do = torch.randn(B, H, Nq, d, generator=g).to(torch.bfloat16)
    label = f"case {i}: B{B} H{H} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} causal{causal} window{window} sharp{int(sharp)}"
    return q, k, v, do, scale, causal, window, label


@pytest.mark.parametrize("i", range(40))
def test_random_forward(i):
    q, k, v, _, scale, causal, window, label = draw(i)
    o, lse = mi.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, causal=causal,
                         window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(q, k, v, scale, causal, window)
    check_out(to64(o), o_ref, bf16=True, label=label)
    check_lse(to64(lse), lse_ref, label=label)


@pytest.mark.parametrize("i", range(40, 56))
def test_random_backward(i):
    q, k, v, do, scale, causal, window, label = draw(i)
    check_bwd(q, k, v, do, scale, causal, window, label=label)


def draw_decode(i: int):
    """A decode case: batch, heads, head size, split count and window, with
    per-sequence cache lengths (0 to 2000, some sequences empty)."""
    r = np.random.default_rng(2000 + i)
    d = int(r.choice([64, 128]))
    G = int(r.choice([1, 2, 4, 8, 16, 40]))
    Hkv = int(r.integers(1, 3))
    B = int(r.integers(1, 6))
    lens = [int(x) if r.random() > 0.1 else 0 for x in r.integers(1, 2001, size=B)]
    Nk = max(max(lens), 1)
    splits = min(int(r.choice([0, 1, 2, 3, 16, 64])), Nk)  # at most Nk (else EINVAL)
    window = 0 if r.random() < 0.6 else int(r.integers(1, 400))
    ps = int(r.choice([1, 16, 64]))
    scale = float(np.float32(1 / math.sqrt(d)))
    label = (f"decode case {i}: B{B} H{Hkv * G} Hkv{Hkv} d{d} lens{lens} splits{splits} "
             f"window{window} page{ps}")
    return r, B, Hkv * G, Hkv, d, lens, Nk, splits, window, ps, scale, label


@pytest.mark.parametrize("i", range(24))
def test_random_decode(i):
    """Contiguous caches at full length, the same caches with per-sequence
    lengths, and the same keys in a shuffled page pool, against the oracle."""
    r, B, H, Hkv, d, lens, Nk, splits, window, ps, scale, label = draw_decode(i)
    g = torch.Generator().manual_seed(9000 + i)
    q = torch.randn(B, H, d, generator=g).to(torch.bfloat16)
    kc = torch.randn(B, Hkv, Nk, d, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Hkv, Nk, d, generator=g).to(torch.bfloat16)
    qd, kd, vd = q.to(DEV), kc.to(DEV), vc.to(DEV)
    o, lse = mi.attn_decode(qd, kd, vd, scale=scale, window=window, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_ref(q, kc, vc, scale, window)
    check_out(to64(o), o_ref, bf16=True, label=label + " (full length)")
    check_lse(to64(lse), l_ref, label=label + " (full length)")

    lens_t = torch.as_tensor(lens, dtype=torch.int32)
    o, lse = mi.attn_decode_varlen(qd, kd, vd, lens_t.to(DEV), scale=scale, window=window,
                                   num_splits=splits)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_kvlens_ref(q, kc, vc, lens, scale, window)
    check_out(to64(o), o_ref, bf16=True, label=label + " (lengths)")
    check_lse(to64(lse), l_ref, label=label + " (lengths)")

    # the same keys in pages of ps keys, at shuffled physical positions
    npp = [-(-n // ps) for n in lens]
    num_pages = max(sum(npp), 1)
    perm = r.permutation(num_pages)
    table = np.zeros((B, max(max(npp), 1)), dtype=np.int32)
    kp = torch.zeros(num_pages, Hkv, ps, d, dtype=torch.bfloat16)
    vp = torch.zeros(num_pages, Hkv, ps, d, dtype=torch.bfloat16)
    nxt = 0
    for b in range(B):
        for j in range(npp[b]):
            pg = int(perm[nxt])
            nxt += 1
            table[b, j] = pg
            n = min(ps, lens[b] - j * ps)
            kp[pg, :, :n] = kc[b, :, j * ps:j * ps + n]
            vp[pg, :, :n] = vc[b, :, j * ps:j * ps + n]
    o, lse = mi.attn_decode_paged(qd, kp.to(DEV), vp.to(DEV), torch.from_numpy(table).to(DEV),
                                  lens_t.to(DEV), scale=scale, window=window, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_paged_ref(q, kp, vp, table, lens, ps, scale, window)
    check_out(to64(o), o_ref, bf16=True, label=label + " (paged)")
    check_lse(to64(lse), l_ref, label=label + " (paged)")


@pytest.mark.parametrize("i", range(12))
def test_random_packed(i):
    """Packed documents: random document counts and lengths (documents with
    no queries or no keys included), forward and backward per document."""
    from test_bwd_varlen import case, run as run_packed
    from test_bwd import bounds
    r = np.random.default_rng(3000 + i)
    n_docs = int(r.integers(1, 7))
    lq = [int(x) if r.random() > 0.1 else 0 for x in r.integers(1, 400, size=n_docs)]
    lk = [x if r.random() < 0.6 else int(r.integers(0, 400)) for x in lq]
    d = int(r.choice([64, 128]))
    Hkv = int(r.integers(1, 3))
    H = Hkv * int(r.choice([1, 2, 4]))
    causal = int(r.random() < 0.6)
    window = 0 if r.random() < 0.5 else int(r.integers(1, 200))
    if sum(lq) == 0 or sum(lk) == 0:
        lq[0], lk[0] = max(lq[0], 1), max(lk[0], 1)
    q, k, v, do, cu_q, cu_k = case(lq, lk, H, Hkv, d, seed=4000 + i)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse, dq, dk, dv = run_packed(q, k, v, do, cu_q, cu_k, scale, causal, window)
    label = f"packed case {i}: docs {lq}/{lk} H{H} Hkv{Hkv} d{d} causal{causal} window{window}"
    o_ref, l_ref = oracle.attention_varlen_ref(q, k, v, cu_q, cu_k, scale, causal, window)
    check_out(to64(o), o_ref, bf16=True, label=label)
    check_lse(to64(lse), l_ref, label=label)
    for e in range(n_docs):
        qs, qe, ks, ke = int(cu_q[e]), int(cu_q[e + 1]), int(cu_k[e]), int(cu_k[e + 1])
        if qe == qs or ke == ks:
            continue
        sl = lambda t, a, b: t[None, :, a:b]
        refs = oracle.attention_bwd_ref(sl(q, qs, qe), sl(k, ks, ke), sl(v, ks, ke),
                                        sl(do, qs, qe), scale, causal, window, return_terms=True)
        tq, tk, tv = bounds(sl(q, qs, qe), sl(k, ks, ke), sl(v, ks, ke), sl(do, qs, qe),
                            o[None, :, qs:qe].cpu(), scale, refs[3], refs[:3])
        for name, got, ref, tol in (("dq", dq[None, :, qs:qe], refs[0], tq),
                                    ("dk", dk[None, :, ks:ke], refs[1], tk),
                                    ("dv", dv[None, :, ks:ke], refs[2], tv)):
            ratio = np.abs(to64(got) - ref) / tol
            assert ratio.max(initial=0.0) <= 1.0, f"{label} doc {e} {name}: err/bound {ratio.max():.3f}"
