"""Split-K decode parity: HIP split + merge kernels against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import DecodeConfig, PrefillConfig
import exact_io_aware_06_amd as mi
from helpers import check_lse, check_out, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def dcfg(B, H, Hkv, Nk, d, splits, window=0):
    return DecodeConfig("t", B, H, Hkv, Nk, d, splits, float(np.float32(1 / math.sqrt(d))),
                        window=window)


def run(c, q, kc, vc, splits=None):
    o, lse = mi.attn_decode(q.to(DEV), kc.to(DEV), vc.to(DEV), scale=c.scale, window=c.window,
                            num_splits=c.splits if splits is None else splits)
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # B, H, Hkv, Nk, d, splits, window
    (3, 8, 2, 1000, 128, 1, 0),
    (3, 8, 2, 1000, 128, 3, 0),
    (3, 8, 2, 1000, 128, 16, 0),
    (3, 8, 2, 1000, 128, 64, 0),
    (3, 8, 2, 1000, 128, 0, 0),
    (3, 8, 2, 1000, 128, 16, 100),
    (3, 8, 2, 1000, 64, 7, 0),
    (2, 4, 4, 333, 64, 5, 40),     # G = 1
    (2, 32, 1, 517, 128, 4, 0),    # G = 32 (MQA)
    (2, 48, 1, 517, 128, 4, 0),    # G = 48: two head blocks, the second half full
    (1, 64, 1, 300, 64, 3, 30),    # G = 64: two full head blocks
    (2, 66, 2, 200, 128, 0, 0),    # G = 33: a second block of one head
    (2, 8, 2, 100, 128, 64, 0),    # trailing splits are empty
    (2, 8, 2, 1, 128, 1, 0),       # a single cached key
    (1, 8, 2, 129, 128, 2, 0),
]


@pytest.mark.parametrize("B,H,Hkv,Nk,d,splits,window", CASES)
def test_decode_small(B, H, Hkv, Nk, d, splits, window):
    c = dcfg(B, H, Hkv, Nk, d, splits, window)
    q, kc, vc = synth.decode_inputs(c, seed=21)
    o, lse = run(c, q, kc, vc)
    o_ref, l_ref = oracle.decode_ref(q, kc, vc, c.scale, window)
    check_out(to64(o), o_ref, bf16=True, label=str(c))
    check_lse(to64(lse), l_ref, label=str(c))


def test_split_counts_agree():
    c = dcfg(4, 16, 4, 3000, 128, 1)
    q, kc, vc = synth.decode_inputs(c, seed=22)
    outs = [run(c, q, kc, vc, splits=s) for s in (1, 3, 16, 64)]
    for o, lse in outs[1:]:
        check_out(to64(o), to64(outs[0][0]), bf16=True, label="splits")
        assert torch.max(torch.abs(lse - outs[0][1])).item() <= 1e-4


def test_decode_equals_last_row_of_causal_prefill():
    N, d = 700, 128
    pc = PrefillConfig("t", 2, 8, 2, N, N, d, "bf16", 1, 0, float(np.float32(1 / math.sqrt(d))))
    q, k, v = synth.prefill_inputs(pc, seed=23)
    o_p, l_p = mi.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=pc.scale, causal=1)
    q_last = q[:, :, -1].contiguous()
    o_d, l_d = mi.attn_decode(q_last.to(DEV), k.to(DEV), v.to(DEV), scale=pc.scale,
                              num_splits=5)
    torch.cuda.synchronize()
    check_out(to64(o_d), to64(o_p[:, :, -1]), bf16=True, label="decode vs prefill")
    assert torch.max(torch.abs(l_d - l_p[:, :, -1])).item() <= 1e-4
    o_ref, l_ref = oracle.decode_ref(q_last, k, v, pc.scale, 0)
    check_out(to64(o_d), o_ref, bf16=True)
    check_lse(to64(l_d), l_ref)


def test_decode_repeated_runs_bit_identical():
    c = dcfg(4, 16, 4, 4000, 128, 16)
    q, kc, vc = synth.decode_inputs(c, seed=24)
    o1, l1 = run(c, q, kc, vc)
    o2, l2 = run(c, q, kc, vc)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
