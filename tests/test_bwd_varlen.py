"""Backward of packed documents (attn_bwd_varlen) against the oracle.

Each document is the fixed-length backward of its own rows, so every
document is compared with the fp64 backward oracle applied to its slices,
under the same derived element-wise bound as the fixed-length backward
(tests/test_bwd.py). Beyond that: equal-length documents give exactly the
batched backward's bits; changing one document's upstream gradient leaves
every other document's gradients bit-identical; keys of a document with no
queries get zero gradients.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import exact_io_aware_06_amd as mi
from helpers import to64
from synth import inputs as S
from test_bwd import bounds

pytestmark = pytest.mark.gpu

DEV = "cuda"


def case(lq, lk, H, Hkv, d, seed):
    g = torch.Generator().manual_seed(seed)
    f = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16)
    return (f(H, sum(lq), d), f(Hkv, sum(lk), d), f(Hkv, sum(lk), d), f(H, sum(lq), d),
            S.cu_seqlens(lq), S.cu_seqlens(lk))


def run(q, k, v, do, cu_q, cu_k, scale, causal, window):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    cq, ck = torch.from_numpy(cu_q).to(DEV), torch.from_numpy(cu_k).to(DEV)
    mq, mk = int(np.diff(cu_q).max(initial=0)), int(np.diff(cu_k).max(initial=0))
    o, lse = mi.attn_fwd_varlen(qd, kd, vd, cq, ck, mq, scale=scale, causal=causal,
                                window=window)
    dq, dk, dv = mi.attn_bwd_varlen(qd, kd, vd, o, lse, dod, cq, ck, mq, mk, scale=scale,
                                    causal=causal, window=window)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


DOCS = [
    ([300, 1, 129, 64, 200], [300, 1, 129, 64, 200]),
    ([100, 200, 50, 33], [400, 150, 0, 33]),     # cached prefixes; a document with no keys
    ([5, 0, 130, 1], [260, 40, 3, 1]),           # a document with keys but no queries
]


@pytest.mark.parametrize("docs", DOCS)
@pytest.mark.parametrize("d,H,Hkv", [(128, 4, 2), (64, 2, 2)])
@pytest.mark.parametrize("causal,window", [(1, 0), (0, 0), (1, 60)])
def test_bwd_varlen_parity(docs, d, H, Hkv, causal, window):
    lq, lk = docs
    q, k, v, do, cu_q, cu_k = case(lq, lk, H, Hkv, d, seed=sum(lq) + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse, dq, dk, dv = run(q, k, v, do, cu_q, cu_k, scale, causal, window)
    for e in range(len(lq)):
        qs, qe, ks, ke = int(cu_q[e]), int(cu_q[e + 1]), int(cu_k[e]), int(cu_k[e + 1])
        label = f"docs={lq}/{lk} d={d} causal={causal} W={window} doc {e}"
        if ke == ks:
            assert torch.all(dq[:, qs:qe] == 0), label  # no keys: no gradient
            continue
        if qe == qs:
            assert torch.all(dk[:, ks:ke] == 0) and torch.all(dv[:, ks:ke] == 0), label
            continue
        sl = lambda t, a, b: t[None, :, a:b]
        refs = oracle.attention_bwd_ref(sl(q, qs, qe), sl(k, ks, ke), sl(v, ks, ke),
                                        sl(do, qs, qe), scale, causal, window,
                                        return_terms=True)
        tq, tk, tv = bounds(sl(q, qs, qe), sl(k, ks, ke), sl(v, ks, ke), sl(do, qs, qe),
                            o[None, :, qs:qe].cpu(), scale, refs[3], refs[:3])
        for name, got, ref, tol in (("dq", dq[None, :, qs:qe], refs[0], tq),
                                    ("dk", dk[None, :, ks:ke], refs[1], tk),
                                    ("dv", dv[None, :, ks:ke], refs[2], tv)):
            ratio = np.abs(to64(got) - ref) / tol
            assert ratio.max(initial=0.0) <= 1.0, f"{label} {name}: err/bound {ratio.max():.3f}"


@pytest.mark.parametrize("causal,window", [(1, 0), (0, 0)])
def test_bwd_varlen_equal_lengths_match_batched(causal, window):
    B, H, Hkv, N, d = 3, 8, 2, 384, 128
    g = torch.Generator().manual_seed(4)
    f = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16).to(DEV)
    q, k, v, do = f(B, H, N, d), f(B, Hkv, N, d), f(B, Hkv, N, d), f(B, H, N, d)
    o, lse = mi.attn_fwd(q, k, v, scale=0.088, causal=causal, window=window)
    dq, dk, dv = mi.attn_bwd(q, k, v, o, lse, do, scale=0.088, causal=causal, window=window)
    pack = lambda x: x.transpose(0, 1).reshape(x.shape[1], B * N, d).contiguous()
    cu = torch.from_numpy(S.cu_seqlens([N] * B)).to(DEV)
    op, lp = mi.attn_fwd_varlen(pack(q), pack(k), pack(v), cu, cu, N, scale=0.088,
                                causal=causal, window=window)
    pq, pk, pv = mi.attn_bwd_varlen(pack(q), pack(k), pack(v), op, lp, pack(do), cu, cu, N, N,
                                    scale=0.088, causal=causal, window=window)
    torch.cuda.synchronize()
    assert torch.equal(pq, pack(dq)) and torch.equal(pk, pack(dk)) and torch.equal(pv, pack(dv))


def test_bwd_varlen_no_leakage():
    lq = [200, 129, 64, 300]
    q, k, v, do, cu_q, cu_k = case(lq, lq, 8, 2, 128, seed=11)
    a = run(q, k, v, do, cu_q, cu_k, 0.088, 1, 0)[2:]
    e = 2
    do2 = do.clone()
    do2[:, cu_q[e]:cu_q[e + 1]] = torch.randn(8, lq[e], 128).to(torch.bfloat16)
    b = run(q, k, v, do2, cu_q, cu_k, 0.088, 1, 0)[2:]
    inside = torch.zeros(sum(lq), dtype=torch.bool, device=DEV)
    inside[cu_q[e]:cu_q[e + 1]] = True
    for x, y in zip(a, b):
        assert torch.equal(x[:, ~inside], y[:, ~inside])
        assert not torch.equal(x[:, inside], y[:, inside])
