"""The Python binding rejects bad caller-provided buffers before any library call.

Runs on the CPU. The library is replaced by a recorder whose only answers are
workspace sizes, and the tensors are host tensors presented as tensors on
GPU 0 (shape, dtype, device and strides are all the checks read). Each case
must raise ValueError and must not reach an entry point that launches work,
so even a check that regresses cannot launch a kernel from these tests.
"""

import pytest
import torch

import exact_io_aware_06_amd as mi
from exact_io_aware_06_amd import api

GPU0 = torch.device("cuda", 0)
GPU1 = torch.device("cuda", 1)
HOST = torch.device("cpu")


class Fake:
    """A host tensor that reports `device` as its device."""

    def __init__(self, shape, dtype=torch.bfloat16, device=GPU0, transpose=False):
        t = torch.zeros(shape, dtype=dtype)
        if transpose:
            t = t.transpose(-1, -2)
        self._t = t
        self.device = device

    @property
    def shape(self):
        return self._t.shape

    @property
    def dtype(self):
        return self._t.dtype

    @property
    def is_cuda(self):
        return self.device.type == "cuda"

    def dim(self):
        return self._t.dim()

    def is_contiguous(self):
        return self._t.is_contiguous()

    def numel(self):
        return self._t.numel()

    def element_size(self):
        return self._t.element_size()

    def data_ptr(self):
        return 0x1000


class Recorder:
    """Stands in for the library: sizes are answered, every other call is recorded."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append(name)
            if name.endswith("_workspace_bytes"):
                return 4096
            if name == "attn_strerror":
                return b"recorded"
            return 0
        return fn

    def launches(self):
        return [c for c in self.calls if not c.endswith("_workspace_bytes")]


@pytest.fixture
def rec(monkeypatch):
    r = Recorder()
    monkeypatch.setattr(api, "load_library", lambda: r)
    return r


def rejects(rec, fn, *args, **kw):
    with pytest.raises(ValueError):
        fn(*args, **kw)
    assert rec.launches() == [], f"reached the library: {rec.launches()}"


B, H, HKV, NQ, NK, D = 1, 4, 2, 64, 64, 128


def qkv():
    return Fake((B, H, NQ, D)), Fake((B, HKV, NK, D)), Fake((B, HKV, NK, D))


@pytest.mark.parametrize("bad", [
    dict(out=Fake((B, H, NQ, 64))),
    dict(out=Fake((B, H, NQ, D), dtype=torch.float32)),
    dict(out=Fake((B, H, NQ, D), device=HOST)),
    dict(out=Fake((B, H, NQ, D), device=GPU1)),
    dict(out=Fake((B, H, D, NQ), transpose=True)),
    dict(lse=Fake((B, H, NQ + 1), dtype=torch.float32)),
    dict(lse=Fake((B, H, NQ), dtype=torch.bfloat16)),
    dict(lse=Fake((B, H, NQ), dtype=torch.float32, device=HOST)),
])
def test_fwd_rejects_bad_outputs(rec, bad):
    q, k, v = qkv()
    kw = dict(out=Fake((B, H, NQ, D)), lse=Fake((B, H, NQ), dtype=torch.float32))
    kw.update(bad)
    rejects(rec, mi.attn_fwd, q, k, v, causal=True, **kw)


def test_fwd_accepts_good_outputs(rec, monkeypatch):
    # The good case reaches the library (the recorder), which is the point of
    # the comparison: the rejections above are made by the checks.
    monkeypatch.setattr(api, "_stream", lambda dev: None)
    monkeypatch.setattr(torch.cuda, "device", lambda dev: _Null())
    q, k, v = qkv()
    mi.attn_fwd(q, k, v, causal=True, out=Fake((B, H, NQ, D)),
                lse=Fake((B, H, NQ), dtype=torch.float32))
    assert rec.launches() == ["attn_fwd"]


class _Null:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


@pytest.mark.parametrize("bad", [
    dict(out=Fake((B, H, NQ, D), dtype=torch.float32)),
    dict(lse=Fake((B, H, NQ), dtype=torch.float32, device=GPU1)),
])
def test_fp8_rejects_bad_outputs(rec, bad):
    q8 = Fake((B, H, NQ, D), dtype=torch.float8_e4m3fn)
    k8 = Fake((B, HKV, NK, D), dtype=torch.float8_e4m3fn)
    v = Fake((B, HKV, NK, D))
    kw = dict(out=Fake((B, H, NQ, D)), lse=Fake((B, H, NQ), dtype=torch.float32))
    kw.update(bad)
    rejects(rec, mi.attn_fwd_fp8, q8, k8, v, 1.0, 1.0, **kw)


@pytest.mark.parametrize("bad", [
    dict(out=Fake((H, 100, D), device=HOST)),
    dict(lse=Fake((H, 99), dtype=torch.float32)),
])
def test_varlen_rejects_bad_outputs(rec, bad):
    q, k, v = Fake((H, 100, D)), Fake((HKV, 100, D)), Fake((HKV, 100, D))
    cu = Fake((3,), dtype=torch.int32)
    kw = dict(out=Fake((H, 100, D)), lse=Fake((H, 100), dtype=torch.float32))
    kw.update(bad)
    rejects(rec, mi.attn_fwd_varlen, q, k, v, cu, cu, 60, **kw)


DEC_GOOD = lambda: dict(out=Fake((3, H, D)), lse=Fake((3, H), dtype=torch.float32),
                        workspace=Fake((4096,), dtype=torch.uint8))
DEC_BAD = [
    dict(out=Fake((3, H, 64))),
    dict(out=Fake((3, H, D), device=HOST)),
    dict(out=Fake((3, H, D), dtype=torch.float32)),
    dict(lse=Fake((3, H + 1), dtype=torch.float32)),
    dict(lse=Fake((3, H), dtype=torch.float32, device=GPU1)),
    dict(workspace=Fake((4095,), dtype=torch.uint8)),          # one byte short
    dict(workspace=Fake((1023,), dtype=torch.float32)),        # 4092 bytes
    dict(workspace=Fake((4096,), dtype=torch.uint8, device=HOST)),
    dict(workspace=Fake((64, 64), dtype=torch.uint8, transpose=True)),
]


@pytest.mark.parametrize("bad", DEC_BAD)
def test_decode_rejects_bad_buffers(rec, bad):
    kw = DEC_GOOD()
    kw.update(bad)
    rejects(rec, mi.attn_decode, Fake((3, H, D)), Fake((3, HKV, 500, D)),
            Fake((3, HKV, 500, D)), **kw)


@pytest.mark.parametrize("bad", DEC_BAD)
def test_decode_varlen_rejects_bad_buffers(rec, bad):
    kw = DEC_GOOD()
    kw.update(bad)
    rejects(rec, mi.attn_decode_varlen, Fake((3, H, D)), Fake((3, HKV, 500, D)),
            Fake((3, HKV, 500, D)), Fake((3,), dtype=torch.int32), **kw)


@pytest.mark.parametrize("bad", DEC_BAD)
def test_decode_paged_rejects_bad_buffers(rec, bad):
    kw = DEC_GOOD()
    kw.update(bad)
    rejects(rec, mi.attn_decode_paged, Fake((3, H, D)), Fake((40, HKV, 16, D)),
            Fake((40, HKV, 16, D)), Fake((3, 10), dtype=torch.int32),
            Fake((3,), dtype=torch.int32), **kw)


def test_decode_workspace_in_bytes_not_elements(rec, monkeypatch):
    """A float32 workspace of 1024 elements is 4096 bytes: accepted, and the
    byte count (not the element count) is what the library receives."""
    seen = {}

    def splitk(*args):
        seen["ws_bytes"] = args[-2].value
        return 0

    monkeypatch.setattr(api, "_stream", lambda dev: None)
    monkeypatch.setattr(torch.cuda, "device", lambda dev: _Null())
    monkeypatch.setattr(rec, "attn_decode_splitk", splitk, raising=False)
    kw = DEC_GOOD()
    kw["workspace"] = Fake((1024,), dtype=torch.float32)
    mi.attn_decode(Fake((3, H, D)), Fake((3, HKV, 500, D)), Fake((3, HKV, 500, D)), **kw)
    assert seen["ws_bytes"] == 4096


BWD_BAD = [
    dict(dq=Fake((B, H, NQ, D), device=HOST)),
    dict(dq=Fake((B, H, NQ, D), dtype=torch.float32)),
    dict(dk=Fake((B, H, NK, D))),                              # H rows, not Hkv
    dict(dk=Fake((B, HKV, NK, D), device=GPU1)),
    dict(dv=Fake((B, HKV, D, NK), transpose=True)),
    dict(workspace=Fake((4095,), dtype=torch.uint8)),
    dict(workspace=Fake((4096,), dtype=torch.uint8, device=HOST)),
]


@pytest.mark.parametrize("bad", BWD_BAD)
def test_bwd_rejects_bad_buffers(rec, bad):
    q, k, v = qkv()
    o, dout = Fake((B, H, NQ, D)), Fake((B, H, NQ, D))
    lse = Fake((B, H, NQ), dtype=torch.float32)
    kw = dict(dq=Fake((B, H, NQ, D)), dk=Fake((B, HKV, NK, D)), dv=Fake((B, HKV, NK, D)),
              workspace=Fake((4096,), dtype=torch.uint8))
    kw.update(bad)
    rejects(rec, mi.attn_bwd, q, k, v, o, lse, dout, causal=True, **kw)


@pytest.mark.parametrize("bad", BWD_BAD[:2] + BWD_BAD[5:])
def test_bwd_varlen_rejects_bad_buffers(rec, bad):
    q, k, v = Fake((H, 100, D)), Fake((HKV, 100, D)), Fake((HKV, 100, D))
    o, dout = Fake((H, 100, D)), Fake((H, 100, D))
    lse = Fake((H, 100), dtype=torch.float32)
    cu = Fake((3,), dtype=torch.int32)
    kw = dict(dq=Fake((H, 100, D)), dk=Fake((HKV, 100, D)), dv=Fake((HKV, 100, D)),
              workspace=Fake((4096,), dtype=torch.uint8))
    if "dq" in bad:
        bad = {"dq": Fake((H, 100, D), device=bad["dq"].device, dtype=bad["dq"].dtype)}
    kw.update(bad)
    rejects(rec, mi.attn_bwd_varlen, q, k, v, o, lse, dout, cu, cu, 60, 60, causal=True, **kw)
