"""Pins for the fp64 oracle: each test checks it against something other than itself.

* brute force: scalar Python loops (math.exp / math.fsum) over tiny inputs;
* a library routine: torch's own CPU scaled-dot-product attention in float64
  (output, log-sum-exp, and its grouped-query head mapping);
* invariants and closed forms the pages fix: probability rows sum to one
  (softmax normalises by the row sum), V = 1 gives 1, identical keys give
  the mean of the visible values, adding a per-row constant to the scores
  changes nothing but the LSE, replicated K/V heads equal GQA;
* the pages' online-softmax recurrence and the split-K merge as separate
  fp64 models, which must agree with the one-shot definition.
"""

import math
import random

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import visible_mask

RNG = np.random.default_rng(1234)


def rand(*shape):
    return RNG.standard_normal(shape)


# --------------------------------------------------------------------------
# brute force


def brute_force(q, k, v, scale, causal, window):
    """Scalar loops over nested lists; keys visited as explicit index ranges."""
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = H // Hkv
    O = [[[[0.0] * v.shape[3] for _ in range(Nq)] for _ in range(H)] for _ in range(B)]
    L = [[[0.0] * Nq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            g = h // G
            for i in range(Nq):
                pos = i + Nk - Nq
                first = max(0, pos - window) if window else 0
                if causal:
                    last = min(pos, Nk - 1)
                else:
                    last = min(Nk - 1, pos + window) if window else Nk - 1
                keys = list(range(first, last + 1))
                if not keys:
                    L[b][h][i] = -math.inf
                    continue
                sc = [scale * math.fsum(float(q[b, h, i, c]) * float(k[b, g, j, c])
                                        for c in range(d)) for j in keys]
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                den = math.fsum(w)
                for c in range(v.shape[3]):
                    O[b][h][i][c] = math.fsum(w[t] * float(v[b, g, j, c])
                                              for t, j in enumerate(keys)) / den
                L[b][h][i] = mx + math.log(den)
    return np.array(O), np.array(L)


CASES = [
    # (Nq, Nk, d, H, Hkv)
    (1, 1, 1, 1, 1),
    (5, 5, 2, 2, 1),
    (7, 16, 4, 4, 2),
    (16, 16, 8, 4, 4),
    (16, 7, 4, 2, 2),   # Nq > Nk: early rows see nothing under causal
    (3, 12, 8, 4, 1),   # MQA
]


@pytest.mark.parametrize("Nq,Nk,d,H,Hkv", CASES)
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("window", [0, 1, 2, 5])
def test_brute_force(Nq, Nk, d, H, Hkv, causal, window):
    q, k, v = rand(2, H, Nq, d), rand(2, Hkv, Nk, d), rand(2, Hkv, Nk, d)
    scale = 0.7
    o, lse = oracle.attention_ref(q, k, v, scale, causal, window)
    ob, lb = brute_force(q, k, v, scale, causal, window)
    fin = np.isfinite(lb)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.all(lse[~fin] == -np.inf)
    assert np.max(np.abs(lse[fin] - lb[fin]), initial=0) <= 1e-12
    assert np.max(np.abs(o - ob)) <= 1e-12


# --------------------------------------------------------------------------
# library routine: torch CPU attention in float64


@pytest.mark.parametrize("H,Hkv", [(1, 1), (4, 4), (8, 2), (4, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa(H, Hkv, causal):
    Nq = Nk = 37
    d = 16
    q, k, v = rand(2, H, Nq, d), rand(2, Hkv, Nk, d), rand(2, Hkv, Nk, d)
    scale = 0.125
    o, lse = oracle.attention_ref(q, k, v, scale, causal, 0)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ot = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=True)
    assert np.max(np.abs(o - ot.numpy())) <= 1e-12
    G = H // Hkv
    of, lf = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        tq, tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1), 0.0, causal,
        scale=scale)
    assert np.max(np.abs(o - of.numpy())) <= 1e-12
    assert np.max(np.abs(lse - lf.numpy())) <= 1e-12


# --------------------------------------------------------------------------
# invariants and closed forms


@pytest.mark.parametrize("causal,window", [(0, 0), (1, 0), (1, 3), (0, 3)])
def test_probability_rows_sum_to_one(causal, window):
    q, k = rand(1, 2, 24, 8), rand(1, 1, 24, 8)
    for h in range(2):
        P = oracle.softmax_probs(q, k, 0.5, causal, window, b=0, h=h)
        vis = visible_mask(24, 24, causal, window)
        assert np.all(P[~vis] == 0)
        assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-14


@pytest.mark.parametrize("causal,window", [(0, 0), (1, 0), (1, 4), (0, 2)])
def test_v_ones_gives_ones(causal, window):
    q, k = rand(2, 4, 20, 8) * 3, rand(2, 2, 20, 8) * 3
    v = np.ones((2, 2, 20, 8))
    o, _ = oracle.attention_ref(q, k, v, 1.0, causal, window)
    assert np.max(np.abs(o - 1.0)) <= 1e-14


@pytest.mark.parametrize("causal,window", [(0, 0), (1, 0), (1, 5), (0, 5)])
def test_identical_keys_give_visible_mean(causal, window):
    Nq = Nk = 30
    q, v = rand(1, 2, Nq, 8), rand(1, 2, Nk, 8)
    krow = rand(8)
    k = np.broadcast_to(krow, (1, 2, Nk, 8)).copy()
    scale = 0.9
    o, lse = oracle.attention_ref(q, k, v, scale, causal, window)
    for h in range(2):
        for i in range(Nq):
            # the visible set, enumerated without the oracle's mask helper
            keys = [j for j in range(Nk)
                    if (not causal or j <= i)
                    and (window == 0 or (i - window <= j and (causal or j <= i + window)))]
            mean = v[0, h, keys].mean(axis=0)
            s = scale * float(q[0, h, i] @ krow)
            assert np.max(np.abs(o[0, h, i] - mean)) <= 1e-13
            assert abs(lse[0, h, i] - (s + math.log(len(keys)))) <= 1e-13


def test_row_shift_invariance():
    """Adding delta_i to every score of row i leaves O and shifts LSE by delta_i."""
    Nq = Nk = 25
    d = 8
    q, k, v = rand(1, 2, Nq, d), rand(1, 2, Nk, d), rand(1, 2, Nk, d)
    k[..., d - 1] = 1.0
    q[..., d - 1] = 0.0
    scale = 0.6
    o0, l0 = oracle.attention_ref(q, k, v, scale, True, 0)
    delta = rand(1, 2, Nq) * 5
    q2 = q.copy()
    q2[..., d - 1] = delta
    o1, l1 = oracle.attention_ref(q2, k, v, scale, True, 0)
    assert np.max(np.abs(o1 - o0)) <= 1e-12
    assert np.max(np.abs(l1 - (l0 + scale * delta))) <= 1e-12


@pytest.mark.parametrize("H,Hkv", [(8, 2), (8, 1), (6, 3)])
def test_gqa_equals_replicated_heads(H, Hkv):
    q, k, v = rand(2, H, 17, 8), rand(2, Hkv, 19, 8), rand(2, Hkv, 19, 8)
    G = H // Hkv
    o, lse = oracle.attention_ref(q, k, v, 0.4, True, 6)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    o2, lse2 = oracle.attention_ref(q, kr, vr, 0.4, True, 6)
    assert np.array_equal(o, o2)
    assert np.array_equal(lse, lse2)


def test_empty_rows_give_zero_and_minus_inf():
    # Nq > Nk causal: row i sits at position i - 4; rows 0..3 see nothing.
    q, k, v = rand(1, 1, 10, 4), rand(1, 1, 6, 4), rand(1, 1, 6, 4)
    o, lse = oracle.attention_ref(q, k, v, 1.0, True, 0)
    assert np.all(o[0, 0, :4] == 0)
    assert np.all(lse[0, 0, :4] == -np.inf)
    assert np.all(np.isfinite(lse[0, 0, 4:]))


@pytest.mark.parametrize("Nq,Nk,causal,window", [
    (64, 64, 1, 0), (64, 64, 1, 9), (50, 64, 1, 9), (64, 64, 0, 9), (64, 64, 0, 0),
])
def test_zero_queries_count_visible_keys(Nq, Nk, causal, window):
    """q = 0 makes every score 0, so LSE_i = ln |visible keys of row i|."""
    q = np.zeros((1, 1, Nq, 8))
    k, v = rand(1, 1, Nk, 8), rand(1, 1, Nk, 8)
    _, lse = oracle.attention_ref(q, k, v, 1.0, causal, window)
    for i in range(Nq):
        p = i + Nk - Nq
        if causal:
            n = min(p + 1, window + 1) if window else p + 1
        else:
            lo = max(0, p - window) if window else 0
            hi = min(Nk - 1, p + window) if window else Nk - 1
            n = hi - lo + 1
        assert round(math.exp(lse[0, 0, i])) == n


# --------------------------------------------------------------------------
# the pages' algorithms as independent models


@pytest.mark.parametrize("causal,window", [(0, 0), (1, 0), (1, 7), (0, 7)])
def test_online_softmax_recurrence_equals_definition(causal, window):
    rnd = random.Random(7)
    Nq, Nk, d = 21, 53, 8
    q, k, v = rand(Nq, d) * 2, rand(Nk, d) * 2, rand(Nk, d)
    vis = visible_mask(Nq, Nk, causal, window)
    o_ref, l_ref = oracle.attention_ref(q[None, None], k[None, None], v[None, None],
                                        0.8, causal, window)
    for _ in range(5):
        sizes, left = [], Nk
        while left:
            s = min(left, rnd.choice([0, 1, 3, 8, 16, 64]))
            sizes.append(s)
            left -= s
        o, lse = oracle.online_softmax_model(q, k, v, 0.8, vis, sizes)
        fin = np.isfinite(l_ref[0, 0])
        assert np.array_equal(fin, np.isfinite(lse))
        assert np.max(np.abs(o - o_ref[0, 0])) <= 1e-12
        assert np.max(np.abs(lse[fin] - l_ref[0, 0][fin]), initial=0) <= 1e-12


@pytest.mark.parametrize("window", [0, 10])
def test_split_merge_equals_unsplit_decode(window):
    rnd = random.Random(3)
    B, H, Hkv, Nk, d = 2, 4, 2, 45, 8
    q, kc, vc = rand(B, H, d), rand(B, Hkv, Nk, d), rand(B, Hkv, Nk, d)
    o_ref, l_ref = oracle.decode_ref(q, kc, vc, 0.5, window)
    for nsplit in (1, 3, 7, 45, 60):
        cuts = sorted(rnd.randint(0, Nk) for _ in range(nsplit - 1))
        edges = [0] + cuts + [Nk]
        bounds = list(zip(edges[:-1], edges[1:]))    # may contain empty splits
        o_s, lse_s = oracle.split_partials_ref(q, kc, vc, 0.5, window, bounds)
        o, lse = oracle.merge_ref(o_s, lse_s)
        assert np.max(np.abs(o - o_ref)) <= 1e-12
        assert np.max(np.abs(lse - l_ref)) <= 1e-12


def test_decode_is_last_row_of_causal_prefill():
    B, H, Hkv, N, d = 2, 4, 1, 33, 8
    q, k, v = rand(B, H, N, d), rand(B, Hkv, N, d), rand(B, Hkv, N, d)
    o, lse = oracle.attention_ref(q, k, v, 0.3, True, 0)
    od, ld = oracle.decode_ref(q[:, :, -1], k, v, 0.3, 0)
    assert np.max(np.abs(od - o[:, :, -1])) <= 1e-13
    assert np.max(np.abs(ld - lse[:, :, -1])) <= 1e-13
    ow, lw = oracle.attention_ref(q, k, v, 0.3, True, 5)
    odw, ldw = oracle.decode_ref(q[:, :, -1], k, v, 0.3, 5)
    assert np.max(np.abs(odw - ow[:, :, -1])) <= 1e-13


def test_row_samples_match_full():
    q, k, v = rand(2, 4, 40, 8), rand(2, 2, 40, 8), rand(2, 2, 40, 8)
    o, lse = oracle.attention_ref(q, k, v, 0.5, True, 11)
    rows = [0, 3, 39, 17]
    os_, ls = oracle.attention_rows_ref(q, k, v, 0.5, True, 11, 1, 3, rows)
    assert np.array_equal(os_, o[1, 3, rows])
    assert np.array_equal(ls, lse[1, 3, rows])
    od, ld = oracle.decode_ref(q[:, :, -1], k, v, 0.5, 0)
    odr, ldr = oracle.decode_rows_ref(q[:, :, -1], k, v, 0.5, 0, 1, [2, 0])
    assert np.max(np.abs(odr - od[1, [2, 0]])) <= 1e-15


def test_row_blocking_does_not_change_results(monkeypatch):
    import oracle.attention as A
    q, k, v = rand(1, 2, 50, 8), rand(1, 1, 50, 8), rand(1, 1, 50, 8)
    o, lse = A.attention_ref(q, k, v, 0.5, True, 0)
    monkeypatch.setattr(A, "_ROW_BLOCK_ELEMS", 7 * 50)
    o2, lse2 = A.attention_ref(q, k, v, 0.5, True, 0)
    assert np.max(np.abs(o - o2)) <= 1e-15 and np.max(np.abs(lse - lse2)) <= 1e-15
