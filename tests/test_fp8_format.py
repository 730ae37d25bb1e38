"""The FP8 inputs the oracle widens: torch's float8_e4m3fn decoding of every
one of the 256 codes against the OCP E4M3 definition (1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits, subnormals at exponent 0, no infinities,
S.1111.111 is NaN), and the per-tensor quantizer's round trip."""

import math

import numpy as np
import torch

from synth import inputs as S


def ocp_e4m3(code: int) -> float:
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    v = math.ldexp(m, -9) if e == 0 else math.ldexp(1 + m / 8, e - 7)
    return -v if s else v


def test_every_code_decodes_as_defined():
    got = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = np.array([ocp_e4m3(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.nanmax(want) == 448.0 and min(v for v in want if v > 0) == 2.0 ** -9


def test_quantizer_round_trip():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(4, 1000, generator=g) * 3
    x8, ds = S.quantize_fp8(x)
    assert x8.dtype == torch.float8_e4m3fn
    back = x8.to(torch.float64) * ds
    assert torch.isfinite(back).all()
    assert float(back.abs().max()) <= float(x.abs().max()) * (1 + 2 ** -4)
    # normal range: relative error <= 2^-4 (3 mantissa bits, round to nearest)
    big = x.abs() >= 2.0 ** -6 * ds
    rel = ((back - x.double()).abs() / x.double().abs())[big]
    assert float(rel.max()) <= 2.0 ** -4 + 1e-12
