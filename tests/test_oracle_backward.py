"""Pins for the backward oracle (CPU only).

* a library routine: torch autograd in float64 through the explicit
  softmax(scale * Q K^T + mask) V, with GQA by repeating K/V heads (autograd
  then sums the group's gradients itself);
* finite differences: the directional derivative of L = sum(O * dO), with O
  from the (already pinned) forward oracle, by central differences;
* closed forms: the gradients of a key sum to zero over keys (softmax rows
  are shift-invariant), the value gradients sum to the sum of dO over rows
  that see a key, a row that sees one key has dq = 0, and keys no row sees
  get zero gradients.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import attention_ref, visible_mask
from oracle.backward import attention_bwd_ref

RNG = np.random.default_rng(777)


def autograd_ref(q, k, v, do, scale, causal, window):
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = H // Hkv
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    kr = kt.repeat_interleave(G, dim=1)
    vr = vt.repeat_interleave(G, dim=1)
    s = torch.matmul(qt, kr.transpose(-1, -2)) * scale
    vis = torch.from_numpy(visible_mask(Nq, Nk, causal, window))
    s = s.masked_fill(~vis, float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = torch.matmul(p, vr)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


SHAPES = [
    # B, H, Hkv, Nq, Nk, d, causal, window
    (1, 2, 2, 9, 9, 4, 0, 0),
    (2, 4, 2, 7, 7, 3, 1, 0),
    (1, 4, 1, 6, 11, 5, 1, 3),
    (1, 2, 1, 8, 8, 2, 0, 2),
    (2, 2, 2, 5, 12, 4, 1, 0),
]


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,window", SHAPES)
def test_bwd_matches_autograd(B, H, Hkv, Nq, Nk, d, causal, window):
    q = RNG.standard_normal((B, H, Nq, d))
    k = RNG.standard_normal((B, Hkv, Nk, d))
    v = RNG.standard_normal((B, Hkv, Nk, d))
    do = RNG.standard_normal((B, H, Nq, d))
    dq, dk, dv = attention_bwd_ref(q, k, v, do, 0.6, causal, window)
    aq, ak, av = autograd_ref(q, k, v, do, 0.6, causal, window)
    for name, x, y in (("dq", dq, aq), ("dk", dk, ak), ("dv", dv, av)):
        assert np.max(np.abs(x - y)) < 1e-12, name


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,window", SHAPES)
def test_bwd_finite_differences(B, H, Hkv, Nq, Nk, d, causal, window):
    q = RNG.standard_normal((B, H, Nq, d))
    k = RNG.standard_normal((B, Hkv, Nk, d))
    v = RNG.standard_normal((B, Hkv, Nk, d))
    do = RNG.standard_normal((B, H, Nq, d))
    scale = 0.45
    dq, dk, dv = attention_bwd_ref(q, k, v, do, scale, causal, window)

    def loss(qq, kk, vv):
        o, _ = attention_ref(qq, kk, vv, scale, causal, window)
        return float(np.sum(o * do))

    eps = 1e-6
    for which, grad in (("q", dq), ("k", dk), ("v", dv)):
        u = RNG.standard_normal(grad.shape)
        args_p = {"q": q, "k": k, "v": v}
        args_m = dict(args_p)
        args_p[which] = args_p[which] + eps * u
        args_m[which] = args_m[which] - eps * u
        fd = (loss(args_p["q"], args_p["k"], args_p["v"])
              - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
        an = float(np.sum(grad * u))
        assert abs(fd - an) < 1e-6 * max(1.0, abs(an)), (which, fd, an)


@pytest.mark.parametrize("causal,window", [(1, 0), (0, 0), (1, 4)])
def test_bwd_closed_forms(causal, window):
    B, H, Hkv, N, d = 1, 4, 2, 10, 6
    q = RNG.standard_normal((B, H, N, d))
    k = RNG.standard_normal((B, Hkv, N, d))
    v = RNG.standard_normal((B, Hkv, N, d))
    do = RNG.standard_normal((B, H, N, d))
    dq, dk, dv = attention_bwd_ref(q, k, v, do, 0.5, causal, window)
    # every row sees at least itself: softmax shift invariance => sum_j dS_ij = 0
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-12
    # P rows sum to one => sum_j dV_j = sum over the group's rows of dO
    want = do.reshape(B, Hkv, H // Hkv, N, d).sum(axis=(2, 3))
    assert np.max(np.abs(dv.sum(axis=2) - want)) < 1e-12
    if causal:  # row 0 sees only key 0: its softmax is constant
        assert np.max(np.abs(dq[:, :, 0])) == 0.0


def test_bwd_unseen_keys_get_zero_gradient():
    # Nq < Nk with a window: keys before the first query's window are unseen
    q = RNG.standard_normal((1, 2, 4, 3))
    k = RNG.standard_normal((1, 1, 12, 3))
    v = RNG.standard_normal((1, 1, 12, 3))
    do = RNG.standard_normal((1, 2, 4, 3))
    dq, dk, dv = attention_bwd_ref(q, k, v, do, 0.5, True, 2)
    seen = visible_mask(4, 12, True, 2).any(axis=0)
    assert np.all(dk[0, 0, ~seen] == 0) and np.all(dv[0, 0, ~seen] == 0)
    assert np.all(np.abs(dv[0, 0, seen]).sum(axis=-1) > 0)


def test_bwd_empty_rows():
    # Nq > Nk under causal: the leading rows see nothing and get dq = 0
    q = RNG.standard_normal((1, 1, 6, 3))
    k = RNG.standard_normal((1, 1, 3, 3))
    v = RNG.standard_normal((1, 1, 3, 3))
    do = RNG.standard_normal((1, 1, 6, 3))
    dq, dk, dv = attention_bwd_ref(q, k, v, do, 0.5, True, 0)
    assert np.all(dq[0, 0, :3] == 0)
    # rows 3.. see keys 0..: compare against the definition restricted to them
    dq2, dk2, dv2 = attention_bwd_ref(q[:, :, 3:], k, v, do[:, :, 3:], 0.5, True, 0)
    assert np.max(np.abs(dq[:, :, 3:] - dq2)) < 1e-14
    assert np.max(np.abs(dk - dk2)) < 1e-14 and np.max(np.abs(dv - dv2)) < 1e-14
