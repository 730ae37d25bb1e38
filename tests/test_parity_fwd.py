"""Forward parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Small shapes are compared element by element over every output; they span
several query and key tiles with ragged tails, Nq != Nk (including rows that
see no key), GQA/MQA, causal, windowed and unmasked attention. The five
fp32 and d = 64 workloads are compared on every output here, the other
full-size workloads and the points of the causal context sweep in
test_full_size.py.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import PrefillConfig
import exact_io_aware_06_amd as mi
from helpers import check_lse, check_out, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def cfg(B, H, Hkv, Nq, Nk, d, causal, window, dtype="bf16", scale=None, mult=1.0):
    s = float(np.float32(1 / math.sqrt(d))) if scale is None else scale
    return PrefillConfig("t", B, H, Hkv, Nq, Nk, d, dtype, causal, window, s, qk_mult=mult)


def run_gpu(c, q, k, v):
    o, lse = mi.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=c.scale, causal=c.causal,
                         window=c.window)
    torch.cuda.synchronize()
    return o, lse


SMALL = [
    # B, H, Hkv, Nq, Nk, d, causal, window
    (1, 4, 2, 300, 300, 128, 1, 0),
    (1, 4, 2, 300, 300, 128, 0, 0),
    (2, 4, 4, 257, 257, 64, 1, 0),
    (2, 4, 4, 257, 257, 64, 0, 0),
    (1, 4, 1, 200, 333, 128, 1, 0),   # fewer queries than keys
    (1, 2, 2, 333, 200, 64, 1, 0),    # more queries than keys: leading rows see nothing
    (1, 2, 2, 333, 200, 128, 1, 0),
    (1, 4, 2, 390, 390, 128, 1, 50),  # causal sliding window
    (1, 4, 2, 390, 390, 64, 1, 50),
    (1, 4, 2, 390, 390, 64, 0, 37),   # two-sided window
    (1, 4, 2, 390, 390, 128, 0, 37),
    (1, 8, 1, 129, 129, 128, 1, 0),   # MQA; one row spills into a second query tile
    (1, 2, 2, 1, 1, 64, 1, 0),
    (1, 2, 1, 5, 700, 128, 0, 0),     # few queries, many keys
    (3, 6, 3, 64, 64, 64, 1, 3),
    (1, 40, 1, 130, 130, 128, 1, 0),  # 40 query heads on one K/V head
]


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,window", SMALL)
def test_small_bf16(B, H, Hkv, Nq, Nk, d, causal, window):
    c = cfg(B, H, Hkv, Nq, Nk, d, causal, window)
    q, k, v = synth.prefill_inputs(c, seed=11)
    o, lse = run_gpu(c, q, k, v)
    o_ref, lse_ref = oracle.attention_ref(q, k, v, c.scale, causal, window)
    check_out(to64(o), o_ref, bf16=True, label=str(c))
    check_lse(to64(lse), lse_ref, label=str(c))


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,window", SMALL[:12])
def test_small_f32(B, H, Hkv, Nq, Nk, d, causal, window):
    c = cfg(B, H, Hkv, Nq, Nk, d, causal, window, dtype="f32")
    q, k, v = synth.prefill_inputs(c, seed=12)
    o, lse = run_gpu(c, q, k, v)
    o_ref, lse_ref = oracle.attention_ref(q, k, v, c.scale, causal, window)
    check_out(to64(o), o_ref, bf16=False, label=str(c))
    check_lse(to64(lse), lse_ref, label=str(c))


def test_empty_key_range_gives_zero_and_minus_inf():
    c = cfg(1, 2, 1, 77, 0, 128, 0, 0)
    q, k, v = synth.prefill_inputs(c, seed=4)
    o, lse = run_gpu(c, q, k, v)
    assert torch.all(o.float() == 0)
    assert torch.all(torch.isneginf(lse))


def test_lse_may_be_omitted():
    c = cfg(1, 2, 1, 100, 100, 64, 1, 0)
    q, k, v = synth.prefill_inputs(c, seed=3)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o_ref, _ = mi.attn_fwd(qd, kd, vd, scale=c.scale, causal=1)
    out = torch.empty_like(qd)
    lib = mi.load_library()
    import ctypes
    st = lib.attn_fwd(ctypes.c_void_p(qd.data_ptr()), ctypes.c_void_p(kd.data_ptr()),
                      ctypes.c_void_p(vd.data_ptr()), ctypes.c_void_p(out.data_ptr()), None,
                      1, 2, 1, 100, 100, 64, ctypes.c_float(c.scale), 1, 0,
                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(out, o_ref)


@pytest.mark.parametrize("growth", [20.0, 60.0, 200.0])
@pytest.mark.parametrize("causal", [0, 1])
def test_rising_scores(growth, causal):
    """Scores that rise along the keys by `growth` over the row: every row's
    maximum keeps growing, so the lazily moved reference maximum is moved
    again and again (from one move per few tiles up to one per tile)."""
    B, H, Hkv, N, d = 1, 2, 1, 1000, 128
    g = torch.Generator().manual_seed(int(growth) + causal)
    ramp = torch.linspace(0.0, 1.0, N)[None, None, :, None]
    q = (1.0 + 0.1 * torch.randn(B, H, N, d, generator=g)).to(torch.bfloat16)
    k = (ramp * (growth / d) + 0.05 * torch.randn(B, Hkv, N, d, generator=g) / d).to(torch.bfloat16)
    v = torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16)
    c = cfg(B, H, Hkv, N, N, d, causal, 0, scale=1.0)
    o, lse = run_gpu(c, q, k, v)
    o_ref, lse_ref = oracle.attention_ref(q, k, v, 1.0, causal, 0)
    check_out(to64(o), o_ref, bf16=True, label=f"growth={growth} causal={causal}")
    check_lse(to64(lse), lse_ref, label=f"growth={growth} causal={causal}")


@pytest.mark.parametrize("jump", [30.0, 100.0, 400.0])
@pytest.mark.parametrize("causal,window", [(1, 0), (0, 0), (1, 300), (0, 170)])
def test_score_jump(jump, causal, window):
    """Scores jump by `jump` at keys 517 and 700 (not on a tile edge), so a
    tile's exponentials taken against the old reference maximum overflow
    (to infinity for the larger jumps) and the tile is redone against a new
    one; with a window, some rows start with no reference at all."""
    B, H, Hkv, N, d = 1, 2, 1, 900, 128
    g = torch.Generator().manual_seed(int(jump) + 7 * causal + window)
    step = (torch.arange(N) >= 517).float() + (torch.arange(N) >= 700).float()
    q = (1.0 + 0.1 * torch.randn(B, H, N, d, generator=g)).to(torch.bfloat16)
    k = (step[None, None, :, None] * (jump / d)
         + 0.3 * torch.randn(B, Hkv, N, d, generator=g) / math.sqrt(d)).to(torch.bfloat16)
    v = torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16)
    c = cfg(B, H, Hkv, N, N, d, causal, window, scale=1.0)
    o, lse = run_gpu(c, q, k, v)
    o_ref, lse_ref = oracle.attention_ref(q, k, v, 1.0, causal, window)
    label = f"jump={jump} causal={causal} window={window}"
    check_out(to64(o), o_ref, bf16=True, label=label)
    check_lse(to64(lse), lse_ref, label=label)


# ---------------------------------------------------------------- workloads


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_workload_fp32_single_head(seed):
    c = synth.CONFIGS["f32_n256_d64"]
    q, k, v = synth.prefill_inputs(c, seed)
    o, lse = run_gpu(c, q, k, v)
    o_ref, lse_ref = oracle.attention_ref(q, k, v, c.scale, c.causal, c.window)
    check_out(to64(o), o_ref, bf16=False, label="f32_n256_d64")
    check_lse(to64(lse), lse_ref, label="f32_n256_d64")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_workload_causal_prefill_d64(seed):
    c = synth.CONFIGS["causal_b4_h16_n2048_d64"]
    q, k, v = synth.prefill_inputs(c, seed)
    o, lse = run_gpu(c, q, k, v)
    o_ref, lse_ref = oracle.attention_ref(q, k, v, c.scale, c.causal, c.window)
    check_out(to64(o), o_ref, bf16=True, label="causal_b4_h16_n2048_d64")
    check_lse(to64(lse), lse_ref, label="causal_b4_h16_n2048_d64")


def sample_rows(N, rng, extra=()):
    base = {0, 1, 2, 63, 64, 127, 128, 129, N // 2, N - 129, N - 128, N - 2, N - 1, *extra}
    base |= set(rng.integers(0, N, 12).tolist())
    return sorted(r for r in base if 0 <= r < N)


def check_sampled(c, q, k, v, o, lse, heads, rows_fn, seed):
    rng = np.random.default_rng(seed)
    og, lg = o.float().cpu(), lse.cpu()
    assert torch.isfinite(og).all()
    for b in range(c.B):
        for h in heads:
            rows = rows_fn(rng)
            o_ref, l_ref = oracle.attention_rows_ref(q, k, v, c.scale, c.causal, c.window,
                                                     b, h, rows)
            check_out(og[b, h, rows].double().numpy(), o_ref, bf16=True, label=f"{c.name} h{h}")
            check_lse(lg[b, h, rows].double().numpy(), l_ref, label=f"{c.name} h{h}")


def test_repeated_runs_bit_identical():
    c = synth.CONFIGS["causal_gqa_n8192_d128"].with_(H=8, Hkv=2, Nq=2048, Nk=2048)
    q, k, v = synth.prefill_inputs(c, 5)
    o1, l1 = run_gpu(c, q, k, v)
    o2, l2 = run_gpu(c, q, k, v)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
