"""Comparison helpers for GPU-vs-oracle parity tests.

Tolerances (GPU output widened exactly to float64, compared with the
unrounded float64 oracle):
  fp32 O      max-abs <= 1e-5
  bf16 O      max-abs <= 2e-2, mean-abs <= 2e-3
  LSE         max-abs <= 1e-3 on finite entries; -inf entries exactly -inf
"""

import numpy as np

TOL_F32_MAX = 1e-5
TOL_BF16_MAX = 2e-2
TOL_BF16_MEAN = 2e-3
TOL_LSE = 1e-3


def to64(t):
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def check_lse(lse_gpu, lse_ref, label=""):
    lg = np.asarray(lse_gpu, dtype=np.float64)
    lr = np.asarray(lse_ref, dtype=np.float64)
    inf_ref = np.isneginf(lr)
    assert np.array_equal(np.isneginf(lg), inf_ref), f"{label}: -inf pattern of LSE differs"
    fin = ~inf_ref
    assert np.all(np.isfinite(lg[fin])), f"{label}: non-finite LSE where oracle is finite"
    err = np.max(np.abs(lg[fin] - lr[fin]), initial=0.0)
    assert err <= TOL_LSE, f"{label}: LSE max-abs {err:.3e} > {TOL_LSE}"
    return err


def check_out(o_gpu, o_ref, bf16=True, label=""):
    og = np.asarray(o_gpu, dtype=np.float64)
    orf = np.asarray(o_ref, dtype=np.float64)
    assert og.shape == orf.shape, f"{label}: shape {og.shape} vs {orf.shape}"
    assert np.all(np.isfinite(og)), f"{label}: non-finite output"
    diff = np.abs(og - orf)
    mx, mean = float(diff.max(initial=0.0)), float(diff.mean()) if diff.size else 0.0
    if bf16:
        assert mx <= TOL_BF16_MAX, f"{label}: bf16 O max-abs {mx:.3e} > {TOL_BF16_MAX}"
        assert mean <= TOL_BF16_MEAN, f"{label}: bf16 O mean-abs {mean:.3e} > {TOL_BF16_MEAN}"
    else:
        assert mx <= TOL_F32_MAX, f"{label}: fp32 O max-abs {mx:.3e} > {TOL_F32_MAX}"
    return mx, mean
