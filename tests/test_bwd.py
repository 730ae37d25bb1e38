"""Backward parity: HIP dq, dk, dv against the fp64 oracle.

The GPU path takes attn_fwd's own O and LSE, as a caller would. The
tolerance is an element-wise bound derived from the arithmetic of the
kernels, evaluated with the oracle's fp64 P and dS:

* P and dS are rounded once to bf16 (relative error <= 2^-8) as matrix-core
  operands, so a product term contributes at most 2^-8 of its magnitude;
  the bound uses 2^-7 (a factor 2 margin for fp32 accumulation over up to
  N terms and for the LSE's own fp32 error);
* D = rowsum(dO * O) uses the stored bf16 O: its error
  |dD_i| <= sum_c |dO_ic| |O_ic - O*_ic| (O* the exact output) enters dS as
  P_ij dD_i;
* dP_ij = dO_i . v_j and D_i are fp32 dot products of d exact products,
  summed in different orders by different units: each is within
  gamma = d 2^-24 of its exact value relative to the sum of |terms|, so
  dP_ij - D_i carries E_ij = gamma (sum_c |dO_ic||v_jc| + sum_c |dO_ic||O_ic|)
  (this is all that is left where the exact dS is 0, e.g. a row that sees a
  single key);
* each output is rounded once to bf16: 2^-8 of its value.

So, per element (sums over visible pairs, and over a group's query heads
for dk / dv):
  |dq - dq*| <= 2^-7 scale sum_j |dS_ij| |k_jc| + scale |dD_i| sum_j P_ij |k_jc|
                + scale sum_j P_ij E_ij |k_jc| + 2^-8 |dq*| + 1e-6
  |dk - dk*| <= sum_h [2^-7 scale sum_i |dS_ij| |q_ic| + scale sum_i P_ij |dD_i| |q_ic|
                       + scale sum_i P_ij E_ij |q_ic|] + 2^-8 |dk*| + 1e-6
  |dv - dv*| <= sum_h 2^-7 sum_i P_ij |dO_ic| + 2^-8 |dv*| + 1e-6
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import exact_io_aware_06_amd as mi
from helpers import to64

pytestmark = pytest.mark.gpu

DEV = "cuda"
U = 2.0 ** -8


def run(q, k, v, do, scale, causal, window):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = mi.attn_fwd(qd, kd, vd, scale=scale, causal=causal, window=window)
    dq, dk, dv = mi.attn_bwd(qd, kd, vd, o, lse, dod, scale=scale, causal=causal,
                             window=window)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def bounds(q, k, v, do, o_gpu, scale, terms, refs):
    """Element-wise tolerances (see the module docstring) for the heads in terms."""
    q64, k64, v64, do64, og = to64(q), to64(k), to64(v), to64(do), to64(o_gpu)
    G = q64.shape[1] // k64.shape[1]
    dq_ref, dk_ref, dv_ref = refs
    tq = np.full(dq_ref.shape, np.inf)
    tk = np.zeros(dk_ref.shape)
    tv = np.zeros(dk_ref.shape)
    for (b, h), t in terms.items():
        P, dS = t["P"], t["dS"]
        kvh = h // G
        o_star = P @ v64[b, kvh]                       # the exact output rows
        ado = np.abs(do64[b, h])
        dD = np.sum(ado * np.abs(og[b, h] - o_star), axis=1)
        gamma = q64.shape[3] * 2.0 ** -24
        PE = P * (gamma * (ado @ np.abs(v64[b, kvh]).T
                           + np.sum(ado * np.abs(og[b, h]), axis=1)[:, None]))
        ak, aq = np.abs(k64[b, kvh]), np.abs(q64[b, h])
        tq[b, h] = (2 * U * scale * (np.abs(dS) @ ak) + scale * dD[:, None] * (P @ ak)
                    + scale * (PE @ ak) + U * np.abs(dq_ref[b, h]) + 1e-6)
        tk[b, kvh] += (2 * U * scale * (np.abs(dS).T @ aq) + scale * (P.T @ (dD[:, None] * aq))
                       + scale * (PE.T @ aq))
        tv[b, kvh] += 2 * U * (P.T @ np.abs(do64[b, h]))
    tk += U * np.abs(dk_ref) + 1e-6
    tv += U * np.abs(dv_ref) + 1e-6
    return tq, tk, tv


def check(q, k, v, do, scale, causal, window, kv_heads=None, label=""):
    """Run forward + backward on the GPU and compare every output of the
    chosen K/V heads' groups with the oracle under the bound. Returns the
    worst |error| / bound and the GPU gradients."""
    o, lse, dq, dk, dv = run(q, k, v, do, scale, causal, window)
    dq_ref, dk_ref, dv_ref, terms = oracle.attention_bwd_ref(
        q, k, v, do, scale, causal, window, return_terms=True, kv_heads=kv_heads)
    tq, tk, tv = bounds(q, k, v, do, o, scale, terms, (dq_ref, dk_ref, dv_ref))
    G = q.shape[1] // k.shape[1]
    kvs = list(range(k.shape[1])) if kv_heads is None else list(kv_heads)
    hs = [kh * G + i for kh in kvs for i in range(G)]
    worst = 0.0
    for name, got, ref, tol, idx in (("dq", dq, dq_ref, tq, hs), ("dk", dk, dk_ref, tk, kvs),
                                     ("dv", dv, dv_ref, tv, kvs)):
        g = to64(got)[:, idx]
        r, t = ref[:, idx], tol[:, idx]
        assert np.all(np.isfinite(g)), f"{label} {name}: non-finite"
        ratio = np.abs(g - r) / t
        worst = max(worst, float(ratio.max(initial=0.0)))
        assert ratio.max(initial=0.0) <= 1.0, (
            f"{label} {name}: |err| / bound = {ratio.max():.3f} at "
            f"{np.unravel_index(ratio.argmax(), ratio.shape)}")
    print(f"{label}: worst |err| / bound = {worst:.3f}")
    return worst, (dq, dk, dv)


def inputs(B, H, Hkv, Nq, Nk, d, seed, mult=1.0):
    g = torch.Generator().manual_seed(seed)
    f = lambda *s: (torch.randn(*s, generator=g) * mult).to(torch.bfloat16)
    return f(B, H, Nq, d), f(B, Hkv, Nk, d), torch.randn(B, Hkv, Nk, d, generator=g).to(
        torch.bfloat16), torch.randn(B, H, Nq, d, generator=g).to(torch.bfloat16)


CASES = [
    # B, H, Hkv, Nq, Nk, d, causal, window
    (1, 4, 2, 300, 300, 128, 1, 0),
    (2, 2, 2, 200, 200, 64, 0, 0),
    (1, 4, 1, 150, 333, 128, 1, 70),
    (1, 2, 2, 77, 200, 128, 1, 0),      # Nq < Nk: a cached prefix
    (1, 2, 1, 260, 100, 64, 1, 0),      # Nq > Nk: leading rows see nothing
    (1, 4, 2, 300, 170, 128, 1, 0),     # the same at d = 128 (LSE = -inf rows in every step)
    (1, 2, 1, 300, 120, 128, 0, 30),    # two-sided window, Nq > Nk: rows 0..149 see nothing
    (1, 4, 4, 129, 129, 128, 0, 40),    # non-causal window
    (2, 8, 2, 256, 256, 128, 1, 0),
    (1, 2, 2, 1, 1, 64, 1, 0),
    (1, 33, 1, 130, 130, 64, 1, 0),     # a group of 33 query heads (one partial sum of 33)
]


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,window", CASES)
def test_bwd_parity(B, H, Hkv, Nq, Nk, d, causal, window):
    q, k, v, do = inputs(B, H, Hkv, Nq, Nk, d, seed=Nq + Nk + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    check(q, k, v, do, scale, causal, window, label=f"{(B, H, Hkv, Nq, Nk, d, causal, window)}")


def test_bwd_sharpened_logits():
    """Peaked softmax rows (logit std 9), as in the sharpened prefill workload."""
    q, k, v, do = inputs(1, 4, 2, 384, 384, 128, seed=3, mult=3.0 * 128 ** -0.25)
    check(q, k, v, do, 1.0, 1, 0, label="sharpened")


def test_bwd_deterministic():
    q, k, v, do = inputs(1, 8, 2, 500, 500, 128, seed=9)
    a = run(q, k, v, do, 0.088, 1, 0)[2:]
    b = run(q, k, v, do, 0.088, 1, 0)[2:]
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_bwd_gqa_equals_replicated_heads():
    """dk, dv of a K/V head shared by G query heads = the sum of the per-head
    gradients of a run with each K/V head replicated G times."""
    q, k, v, do = inputs(1, 8, 2, 256, 256, 128, seed=4)
    _, _, dq1, dk1, dv1 = run(q, k, v, do, 0.088, 1, 0)
    kr, vr = k.repeat_interleave(4, dim=1), v.repeat_interleave(4, dim=1)
    _, _, dq2, dk2, dv2 = run(q, kr, vr, do, 0.088, 1, 0)
    assert torch.equal(dq1, dq2)  # the dq pass does not depend on the grouping
    sk = dk2.float().reshape(1, 2, 4, 256, 128).sum(2)
    sv = dv2.float().reshape(1, 2, 4, 256, 128).sum(2)
    # per-head bf16 rounding before the sum: 4 roundings of 2^-8 relative each
    assert torch.all((dk1.float() - sk).abs() <= 4 * U * dk2.float().reshape(1, 2, 4, 256, 128)
                     .abs().sum(2) + U * sk.abs() + 1e-6)
    assert torch.all((dv1.float() - sv).abs() <= 4 * U * dv2.float().reshape(1, 2, 4, 256, 128)
                     .abs().sum(2) + U * sv.abs() + 1e-6)


def test_bwd_empty_key_range():
    """Nk = 0 for the forward and backward: dq = 0."""
    q = torch.randn(1, 2, 10, 64).to(torch.bfloat16).to(DEV)
    k = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device=DEV)
    o, lse = mi.attn_fwd(q, k, k, scale=0.125, causal=False)
    dq, dk, dv = mi.attn_bwd(q, k, k, o, lse, torch.ones_like(q), scale=0.125)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and dk.numel() == 0


def test_bwd_workload_causal_gqa_one_group():
    """The headline prefill shape (B1 H32 Hkv8 N8192 d128, causal, sharpened):
    every output of one K/V group against the oracle (4 query heads)."""
    c = synth.CONFIGS["causal_gqa_n8192_d128"]
    q, k, v = synth.prefill_inputs(c, 0)
    g = torch.Generator().manual_seed(123)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    worst, _ = check(q, k, v, do, c.scale, c.causal, c.window, kv_heads=[5], label="c3 group 5")
    assert worst <= 1.0


def test_bwd_longest_key_range():
    """The longest key range the C ABI takes for one head (8,388,607 keys at
    d = 128: one head's K / V rows are addressed through 32-bit buffer
    offsets), causal with a 5000-key window, two query heads of one K/V head
    and 32 query rows at the far end: the keys that receive gradients are the
    last ones, at the largest offsets, and every other key's dk / dv is
    compared too (the oracle's are zero). Every output against the oracle."""
    Nk = 0xFFFFFFFF // (128 * 4)
    q, k, v, do = inputs(1, 2, 1, 32, Nk, 128, seed=21)
    scale = float(np.float32(1 / math.sqrt(128)))
    worst, _ = check(q, k, v, do, scale, 1, 5000, label="longest key range")
    assert worst <= 1.0
