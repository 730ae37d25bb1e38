"""Race check of the LDS copy rings: pipelined kernels vs fully fenced ones.

libmiattn_serial.so is the same source compiled with MIATTN_SERIAL_RINGS=1:
every copy into an LDS ring slot (forward K/V rings, dQ K/V ring, dK/dV Q/dO
and statistics ring) has a barrier before it and a wait plus a barrier after
it, and every matrix-core block whose results the vector ALU reads is padded
(the pipelined forward drops that pad after its Q K^T block at d = 128). Only
synchronisation differs, not arithmetic or its order, so the two libraries
must agree bit for bit; a missing wait or barrier, a copy that overwrites a
slot still being read, or too few wait states in the pipelined build would
show up as a difference. The page that warns that silent correctness bugs
are the dangerous kind is "What Lost, and Why" (closing section).

The workloads: the causal GQA prefill at full size (8192 tokens, sharpened),
the causal sliding-window prefill at full size (32768 tokens, window 4096),
the causal d = 64 prefill, packed documents, the fp8 forward, and the
backward at the first two shapes and on packed documents.
"""

import os

import pytest
import torch

import synth
import exact_io_aware_06_amd as mi
from exact_io_aware_06_amd import api
from synth import inputs as S

DEV = "cuda"
SERIAL = os.path.join(os.path.dirname(os.path.abspath(api.__file__)), "libmiattn_serial.so")


def test_serial_library_exports_the_abi():
    """CPU: the race-check build exists next to the release library and
    exports the same entry points."""
    import ctypes
    import re
    assert os.path.exists(SERIAL), "libmiattn_serial.so is not built"
    header = open(os.path.join(os.path.dirname(os.path.dirname(SERIAL)), "include",
                               "miattn.h")).read()
    header = re.sub(r"/\*.*?\*/", "", header, flags=re.S)
    names = set(re.findall(r"(attn_[a-z_0-9]+)\s*\(", header))
    lib = ctypes.CDLL(SERIAL)
    for n in names:
        assert hasattr(lib, n), n


@pytest.fixture(scope="module")
def serial_lib():
    assert os.path.exists(SERIAL), "libmiattn_serial.so is not built"
    with open(SERIAL, "rb") as f, open(api.library_path(), "rb") as g:
        assert f.read() != g.read(), "the race-check library is the release build"
    return api.load_variant(SERIAL)


def both(monkeypatch, serial_lib, fn):
    """fn() with the release library, then with the fenced one."""
    a = fn()
    torch.cuda.synchronize()
    with monkeypatch.context() as m:
        m.setattr(api, "load_library", lambda: serial_lib)
        b = fn()
        torch.cuda.synchronize()
    return a, b


def assert_same(a, b, label):
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x, y), f"{label}: output {i} differs between the pipelined and " \
                                  f"the fenced build"


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["causal_gqa_n8192_d128", "window4096_gqa_n32768_d128",
                                  "causal_b4_h16_n2048_d64"])
def test_forward_bit_identical(monkeypatch, serial_lib, name):
    c = synth.CONFIGS[name]
    q, k, v = synth.prefill_inputs(c, seed=0, device=DEV)
    a, b = both(monkeypatch, serial_lib,
                lambda: mi.attn_fwd(q, k, v, scale=c.scale, causal=c.causal, window=c.window))
    assert_same(a, b, name)


@pytest.mark.gpu
def test_fp8_forward_bit_identical(monkeypatch, serial_lib):
    c = synth.CONFIGS["causal_gqa_n8192_d128"]
    q8, k8, v, qd, kd = S.fp8_prefill_inputs(c, seed=0, device=DEV)
    a, b = both(monkeypatch, serial_lib,
                lambda: mi.attn_fwd_fp8(q8, k8, v, qd, kd, scale=c.scale, causal=1))
    assert_same(a, b, "fp8")


def _packed(seed=0):
    cfg = S.PACKED["packed_24docs_4x8192_d128"]
    lens = cfg.lengths(seed)
    cu = S.cu_seqlens(lens)
    total = int(cu[-1])
    q, k, v = S.packed_inputs(cfg, total, total, seed=seed, device=DEV)
    return cfg, lens, torch.from_numpy(cu).to(DEV), q, k, v, total


@pytest.mark.gpu
def test_packed_forward_bit_identical(monkeypatch, serial_lib):
    cfg, lens, cu, q, k, v, _ = _packed()
    a, b = both(monkeypatch, serial_lib,
                lambda: mi.attn_fwd_varlen(q, k, v, cu, cu, max(lens), scale=cfg.scale,
                                           causal=cfg.causal))
    assert_same(a, b, "packed")


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["causal_gqa_n8192_d128", "window4096_gqa_n32768_d128",
                                  "causal_b4_h16_n2048_d64"])
def test_backward_bit_identical(monkeypatch, serial_lib, name):
    c = synth.CONFIGS[name]
    q, k, v = synth.prefill_inputs(c, seed=1, device=DEV)
    o, lse = mi.attn_fwd(q, k, v, scale=c.scale, causal=c.causal, window=c.window)
    dout = synth.gen_normal(tuple(q.shape[1:]), 1, 4, 0, "bf16", 1.0, DEV)[None].expand(
        q.shape).contiguous()
    a, b = both(monkeypatch, serial_lib,
                lambda: mi.attn_bwd(q, k, v, o, lse, dout, scale=c.scale, causal=c.causal,
                                    window=c.window))
    assert_same(a, b, f"backward {name}")
    del q, k, v, o, lse, dout, a, b
    torch.cuda.empty_cache()


@pytest.mark.gpu
def test_packed_backward_bit_identical(monkeypatch, serial_lib):
    cfg, lens, cu, q, k, v, total = _packed(1)
    o, lse = mi.attn_fwd_varlen(q, k, v, cu, cu, max(lens), scale=cfg.scale, causal=1)
    dout = synth.gen_normal((cfg.H, total, cfg.d), 1, 4, 0, "bf16", 1.0, DEV)
    a, b = both(monkeypatch, serial_lib,
                lambda: mi.attn_bwd_varlen(q, k, v, o, lse, dout, cu, cu, max(lens), max(lens),
                                           scale=cfg.scale, causal=1))
    assert_same(a, b, "packed backward")
