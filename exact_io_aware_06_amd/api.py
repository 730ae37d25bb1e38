"""ctypes binding of libmiattn (argument marshalling only).

Every step of the computation runs in the HIP library. This module checks
tensor dtype/device/shape/contiguity, allocates outputs with torch, and
passes raw pointers plus the current torch stream. If the library is not
built, the first call raises: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmiattn.so"
_lock = threading.Lock()
_lib = None

MIATTN_OK = 0


class MiattnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libmiattn status {status}: {msg}")
        self.status = status


def library_path() -> str:
    return os.environ.get("MIATTN_LIBRARY", os.path.join(_HERE, _LIB_NAME))


def load_library():
    """Load libmiattn.so (once) and declare the C signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        _lib = _open(library_path())
        return _lib


def load_variant(path: str):
    """Load another build of the library (such as the fully fenced race-check
    build libmiattn_serial.so) with the same C signatures declared."""
    with _lock:
        return _open(path)


def _open(path: str):
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
            "from the repository root")
    lib = ctypes.CDLL(path)
    _declare(lib)
    return lib


def _declare(lib):
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    fwd_args = [P, P, P, P, P, I, I, I, I, I, I, F, I, I, P]
    lib.attn_fwd.argtypes = fwd_args
    lib.attn_fwd.restype = I
    lib.attn_fwd_f32.argtypes = fwd_args
    lib.attn_fwd_f32.restype = I
    lib.attn_fwd_fp8.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, F, F, I, I, P]
    lib.attn_fwd_fp8.restype = I
    lib.attn_fwd_tile_counts.argtypes = fwd_args[:-1] + [P, P]
    lib.attn_fwd_tile_counts.restype = I
    varlen_args = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, I]
    lib.attn_fwd_varlen.argtypes = varlen_args + [P]
    lib.attn_fwd_varlen.restype = I
    lib.attn_fwd_varlen_tile_counts.argtypes = varlen_args + [P, P]
    lib.attn_fwd_varlen_tile_counts.restype = I
    lib.attn_decode_splitk_varlen.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, I, I, P,
                                              S, P]
    lib.attn_decode_splitk_varlen.restype = I
    lib.attn_decode_paged.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, P,
                                      S, P]
    lib.attn_decode_paged.restype = I
    lib.attn_bwd_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.attn_bwd_workspace_bytes.restype = S
    lib.attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, P, S, P]
    lib.attn_bwd.restype = I
    lib.attn_bwd_varlen.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I,
                                    F, I, I, P, S, P]
    lib.attn_bwd_varlen.restype = I
    lib.attn_fwd_tile_shape.argtypes = [I, I, ctypes.POINTER(I), ctypes.POINTER(I)]
    lib.attn_fwd_tile_shape.restype = I
    lib.attn_decode_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.attn_decode_workspace_bytes.restype = S
    lib.attn_decode_num_splits.argtypes = [I, I, I, I]
    lib.attn_decode_num_splits.restype = I
    lib.attn_decode_splitk.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I, P, S, P]
    lib.attn_decode_splitk.restype = I
    lib.attn_decode_splitk_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I, P]
    lib.attn_decode_splitk_noalloc.restype = I
    lib.attn_calib_mfma.argtypes = [I, I, P, P]
    lib.attn_calib_mfma.restype = I
    lib.attn_calib_read.argtypes = [P, S, P, I, P]
    lib.attn_calib_read.restype = I
    lib.attn_strerror.argtypes = [I]
    lib.attn_strerror.restype = ctypes.c_char_p


def _check(status: int):
    if status != MIATTN_OK:
        msg = load_library().attn_strerror(status).decode()
        raise MiattnError(status, msg)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() > 0 else 0)


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_buffer(t, shape, dtype, device, name):
    """A caller-provided output buffer must have exactly this shape and dtype,
    live on `device` and be contiguous (the kernels write it in full)."""
    _require(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, "
             f"got {tuple(t.shape)}")
    _require(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _require(t.device == device, f"{name} must be on {device}, got {t.device}")
    _require(t.is_contiguous(), f"{name} must be contiguous")


def _workspace(workspace, nbytes, device):
    """The caller's workspace (checked: on `device`, contiguous, at least
    `nbytes` bytes) or a new one. Returns (tensor, its size in bytes)."""
    import torch
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _require(workspace.device == device, f"workspace must be on {device}, got {workspace.device}")
    _require(workspace.is_contiguous(), "workspace must be contiguous")
    size = workspace.numel() * workspace.element_size()
    _require(size >= nbytes, f"workspace holds {size} bytes, {nbytes} needed")
    return workspace, size


def fwd_tile_shape(d: int, is_f32: bool = False):
    lib = load_library()
    bm, bn = ctypes.c_int(), ctypes.c_int()
    _check(lib.attn_fwd_tile_shape(int(d), int(bool(is_f32)), ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


def _fwd_checks(q, k, v):
    import torch
    _require(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v must be 4-D")
    _require(q.is_cuda and k.device == q.device and v.device == q.device,
             "q, k, v must be on the same GPU")
    _require(q.dtype in (torch.bfloat16, torch.float32), "dtype must be bfloat16 or float32")
    _require(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v dtypes differ")
    _require(q.is_contiguous() and k.is_contiguous() and v.is_contiguous(),
             "q, k, v must be contiguous")
    B, H, Nq, d = q.shape
    _require(k.shape[0] == B and k.shape[3] == d and v.shape == k.shape,
             "k/v must be [B, Hkv, Nk, d] matching q")
    return B, H, k.shape[1], Nq, k.shape[2], d


def attn_fwd(q, k, v, scale=None, causal=False, window=0, out=None, lse=None):
    """Fused attention forward. Returns (O [B,H,Nq,d] like q, LSE [B,H,Nq] fp32).

    bf16 inputs run the bf16 matrix-core kernel, fp32 inputs the fp32 kernel.
    """
    import torch
    B, H, Hkv, Nq, Nk, d = _fwd_checks(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_buffer(out, q.shape, q.dtype, q.device, "out")
    _check_buffer(lse, (B, H, Nq), torch.float32, q.device, "lse")
    lib = load_library()
    fn = lib.attn_fwd if q.dtype == torch.bfloat16 else lib.attn_fwd_f32
    with torch.cuda.device(q.device):
        _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, Nq, Nk, d,
                  ctypes.c_float(scale), int(bool(causal)), int(window), _stream(q.device)))
    return out, lse


def attn_fwd_fp8(q8, k8, v, q_descale, k_descale, scale=None, causal=False, window=0,
                 out=None, lse=None):
    """FP8 forward: q8 [B,H,Nq,d], k8 [B,Hkv,Nk,d] float8_e4m3fn with per-tensor
    descales; v [B,Hkv,Nk,d] bf16. Returns (O bf16 [B,H,Nq,d], LSE fp32 [B,H,Nq])."""
    import torch
    _require(q8.dim() == 4 and k8.dim() == 4 and v.dim() == 4, "q8, k8, v must be 4-D")
    _require(q8.is_cuda and k8.device == q8.device and v.device == q8.device,
             "q8, k8, v must be on the same GPU")
    _require(q8.dtype == torch.float8_e4m3fn and k8.dtype == torch.float8_e4m3fn,
             "q8 and k8 must be float8_e4m3fn")
    _require(v.dtype == torch.bfloat16, "v must be bfloat16")
    _require(q8.is_contiguous() and k8.is_contiguous() and v.is_contiguous(),
             "tensors must be contiguous")
    B, H, Nq, d = q8.shape
    Hkv, Nk = k8.shape[1], k8.shape[2]
    _require(k8.shape[0] == B and k8.shape[3] == d and v.shape == k8.shape,
             "k8/v must be [B, Hkv, Nk, d] matching q8")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q8.device)
    _check_buffer(out, q8.shape, torch.bfloat16, q8.device, "out")
    _check_buffer(lse, (B, H, Nq), torch.float32, q8.device, "lse")
    lib = load_library()
    with torch.cuda.device(q8.device):
        _check(lib.attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv,
                                Nq, Nk, d, ctypes.c_float(scale), ctypes.c_float(q_descale),
                                ctypes.c_float(k_descale), int(bool(causal)), int(window),
                                _stream(q8.device)))
    return out, lse


def fwd_tile_counts(q, k, v, scale=None, causal=False, window=0):
    """attn_fwd (bf16) plus per-work-group (tiles loaded, tiles masked) counts.

    Returns (O, LSE, counts [B, H, ceil(Nq/BM), 2] int32).
    """
    import torch
    B, H, Hkv, Nq, Nk, d = _fwd_checks(q, k, v)
    _require(q.dtype == torch.bfloat16, "tile counts are for the bf16 kernel")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    bm, _ = fwd_tile_shape(d, False)
    nqt = -(-Nq // bm)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    counts = torch.full((B, H, nqt, 2), -1, dtype=torch.int32, device=q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        _check(lib.attn_fwd_tile_counts(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                        B, H, Hkv, Nq, Nk, d, ctypes.c_float(scale),
                                        int(bool(causal)), int(window), _ptr(counts),
                                        _stream(q.device)))
    return out, lse, counts


def _varlen_checks(q, k, v, cu_seqlens_q, cu_seqlens_k):
    import torch
    _require(q.dim() == 3 and k.dim() == 3 and v.shape == k.shape,
             "packed q [H, total_q, d], k/v [Hkv, total_k, d]")
    _require(q.is_cuda and k.device == q.device and v.device == q.device,
             "q, k, v must be on the same GPU")
    _require(q.dtype == torch.bfloat16 and k.dtype == q.dtype and v.dtype == q.dtype,
             "packed attention takes bfloat16")
    _require(q.is_contiguous() and k.is_contiguous() and v.is_contiguous(),
             "q, k, v must be contiguous")
    _require(k.shape[2] == q.shape[2], "head dims differ")
    for cu in (cu_seqlens_q, cu_seqlens_k):
        _require(cu.dim() == 1 and cu.dtype == torch.int32 and cu.device == q.device
                 and cu.is_contiguous(), "cu_seqlens must be contiguous int32 on q's GPU")
    _require(cu_seqlens_q.numel() == cu_seqlens_k.numel() and cu_seqlens_q.numel() >= 1,
             "cu_seqlens_q and cu_seqlens_k must both hold num_seqs + 1 offsets")
    H, total_q, d = q.shape
    return H, k.shape[0], total_q, k.shape[1], d, cu_seqlens_q.numel() - 1


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, scale=None,
                    causal=False, window=0, out=None, lse=None):
    """Packed documents: q [H, total_q, d], k/v [Hkv, total_k, d] bf16.

    cu_seqlens_* are device int32 offsets [num_seqs + 1]; max_seqlen_q bounds
    every document's query count. Returns (O like q, LSE [H, total_q] fp32).
    """
    import torch
    H, Hkv, total_q, total_k, d, ns = _varlen_checks(q, k, v, cu_seqlens_q, cu_seqlens_k)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    _check_buffer(out, q.shape, q.dtype, q.device, "out")
    _check_buffer(lse, (H, total_q), torch.float32, q.device, "lse")
    lib = load_library()
    with torch.cuda.device(q.device):
        _check(lib.attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                   _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), ns, H, Hkv, total_q,
                                   total_k, int(max_seqlen_q), d, ctypes.c_float(scale),
                                   int(bool(causal)), int(window), _stream(q.device)))
    return out, lse


def fwd_varlen_tile_counts(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, scale=None,
                           causal=False, window=0):
    """attn_fwd_varlen plus per-work-group (tiles loaded, tiles masked) counts.

    Returns (O, LSE, counts [num_seqs, H, ceil(max_seqlen_q / BM), 2] int32).
    """
    import torch
    H, Hkv, total_q, total_k, d, ns = _varlen_checks(q, k, v, cu_seqlens_q, cu_seqlens_k)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    bm, _ = fwd_tile_shape(d, False)
    nqt = -(-int(max_seqlen_q) // bm)
    out = torch.empty_like(q)
    lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    counts = torch.full((ns, H, nqt, 2), -1, dtype=torch.int32, device=q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        _check(lib.attn_fwd_varlen_tile_counts(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
            _ptr(cu_seqlens_k), ns, H, Hkv, total_q, total_k, int(max_seqlen_q), d,
            ctypes.c_float(scale), int(bool(causal)), int(window), _ptr(counts),
            _stream(q.device)))
    return out, lse, counts


def decode_workspace_bytes(B, H, Hkv, Nk, d, num_splits=0) -> int:
    return int(load_library().attn_decode_workspace_bytes(B, H, Hkv, Nk, d, num_splits))


def attn_decode(q, k_cache, v_cache, scale=None, window=0, num_splits=0,
                out=None, lse=None, workspace=None):
    """Split-K decode. q [B,H,d] bf16, caches [B,Hkv,Nk,d] bf16.

    Returns (O [B,H,d] bf16, LSE [B,H] fp32).
    """
    import torch
    _require(q.dim() == 3 and k_cache.dim() == 4 and v_cache.shape == k_cache.shape,
             "q [B,H,d], caches [B,Hkv,Nk,d]")
    _require(q.is_cuda and k_cache.device == q.device and v_cache.device == q.device,
             "tensors must be on the same GPU")
    _require(q.dtype == torch.bfloat16 and k_cache.dtype == torch.bfloat16
             and v_cache.dtype == torch.bfloat16, "decode takes bfloat16")
    _require(q.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous(),
             "tensors must be contiguous")
    B, H, d = q.shape
    Hkv, Nk = k_cache.shape[1], k_cache.shape[2]
    _require(k_cache.shape[0] == B and k_cache.shape[3] == d, "cache shape mismatch")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load_library()
    nbytes = int(lib.attn_decode_workspace_bytes(B, H, Hkv, Nk, d, int(num_splits)))
    workspace, ws_bytes = _workspace(workspace, nbytes, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _check_buffer(out, q.shape, torch.bfloat16, q.device, "out")
    _check_buffer(lse, (B, H), torch.float32, q.device, "lse")
    with torch.cuda.device(q.device):
        _check(lib.attn_decode_splitk(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                      _ptr(lse), B, H, Hkv, Nk, d, ctypes.c_float(scale),
                                      int(window), int(num_splits), _ptr(workspace),
                                      ctypes.c_size_t(ws_bytes), _stream(q.device)))
    return out, lse


def attn_decode_splitk_noalloc(q, k_cache, v_cache, out, lse, scale=None, window=0,
                               num_splits=0):
    """attn_decode without a workspace: the library's own per-GPU scratch
    holds the split partials, and nothing is allocated (the caller passes
    out [B,H,d] bf16 and lse [B,H] fp32). Calls that overlap on one GPU race
    on that scratch; issue them on one stream. Returns (out, lse)."""
    import torch
    _require(q.dim() == 3 and k_cache.dim() == 4 and v_cache.shape == k_cache.shape,
             "q [B,H,d], caches [B,Hkv,Nk,d]")
    _require(q.is_cuda and k_cache.device == q.device and v_cache.device == q.device,
             "tensors must be on the same GPU")
    _require(q.dtype == torch.bfloat16 and k_cache.dtype == torch.bfloat16
             and v_cache.dtype == torch.bfloat16, "decode takes bfloat16")
    _require(q.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous(),
             "tensors must be contiguous")
    B, H, d = q.shape
    Hkv, Nk = k_cache.shape[1], k_cache.shape[2]
    _require(k_cache.shape[0] == B and k_cache.shape[3] == d, "cache shape mismatch")
    _check_buffer(out, q.shape, torch.bfloat16, q.device, "out")
    _check_buffer(lse, (B, H), torch.float32, q.device, "lse")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load_library()
    with torch.cuda.device(q.device):
        _check(lib.attn_decode_splitk_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                              _ptr(lse), B, H, Hkv, Nk, d,
                                              ctypes.c_float(scale), int(window),
                                              int(num_splits), _stream(q.device)))
    return out, lse


def attn_decode_varlen(q, k_cache, v_cache, kv_lens, scale=None, window=0, num_splits=0,
                       out=None, lse=None, workspace=None):
    """Split-K decode where sequence b holds kv_lens[b] keys (device int32 [B]).

    q [B,H,d], caches [B,Hkv,Nk,d] bf16. Returns (O [B,H,d] bf16, LSE [B,H] fp32).
    """
    import torch
    _require(q.dim() == 3 and k_cache.dim() == 4 and v_cache.shape == k_cache.shape,
             "q [B,H,d], caches [B,Hkv,Nk,d]")
    _require(q.is_cuda and k_cache.device == q.device and v_cache.device == q.device,
             "tensors must be on the same GPU")
    _require(q.dtype == torch.bfloat16 and k_cache.dtype == torch.bfloat16
             and v_cache.dtype == torch.bfloat16, "decode takes bfloat16")
    _require(q.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous(),
             "tensors must be contiguous")
    B, H, d = q.shape
    Hkv, Nk = k_cache.shape[1], k_cache.shape[2]
    _require(k_cache.shape[0] == B and k_cache.shape[3] == d, "cache shape mismatch")
    _require(kv_lens.shape == (B,) and kv_lens.dtype == torch.int32
             and kv_lens.device == q.device and kv_lens.is_contiguous(),
             "kv_lens must be contiguous int32 [B] on q's GPU")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load_library()
    nbytes = int(lib.attn_decode_workspace_bytes(B, H, Hkv, Nk, d, int(num_splits)))
    workspace, ws_bytes = _workspace(workspace, nbytes, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _check_buffer(out, q.shape, torch.bfloat16, q.device, "out")
    _check_buffer(lse, (B, H), torch.float32, q.device, "lse")
    with torch.cuda.device(q.device):
        _check(lib.attn_decode_splitk_varlen(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                             _ptr(kv_lens), _ptr(out), _ptr(lse), B, H, Hkv, Nk,
                                             d, ctypes.c_float(scale), int(window),
                                             int(num_splits), _ptr(workspace),
                                             ctypes.c_size_t(ws_bytes),
                                             _stream(q.device)))
    return out, lse


def attn_decode_paged(q, k_pages, v_pages, block_table, kv_lens, scale=None, window=0,
                      num_splits=0, out=None, lse=None, workspace=None):
    """Split-K decode over a paged cache.

    q [B,H,d] bf16; k_pages/v_pages [num_pages, Hkv, page_size, d] bf16;
    block_table int32 [B, max_pages] and kv_lens int32 [B], both on q's GPU.
    Returns (O [B,H,d] bf16, LSE [B,H] fp32).
    """
    import torch
    _require(q.dim() == 3 and k_pages.dim() == 4 and v_pages.shape == k_pages.shape,
             "q [B,H,d], pages [num_pages, Hkv, page_size, d]")
    _require(q.is_cuda and k_pages.device == q.device and v_pages.device == q.device,
             "tensors must be on the same GPU")
    _require(q.dtype == torch.bfloat16 and k_pages.dtype == torch.bfloat16
             and v_pages.dtype == torch.bfloat16, "decode takes bfloat16")
    _require(q.is_contiguous() and k_pages.is_contiguous() and v_pages.is_contiguous(),
             "tensors must be contiguous")
    B, H, d = q.shape
    num_pages, Hkv, page_size = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    _require(k_pages.shape[3] == d, "head dim mismatch")
    _require(block_table.dim() == 2 and block_table.shape[0] == B
             and block_table.dtype == torch.int32 and block_table.device == q.device
             and block_table.is_contiguous(), "block_table must be contiguous int32 [B, max_pages]")
    _require(kv_lens.shape == (B,) and kv_lens.dtype == torch.int32
             and kv_lens.device == q.device and kv_lens.is_contiguous(),
             "kv_lens must be contiguous int32 [B] on q's GPU")
    max_pages = block_table.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load_library()
    nbytes = int(lib.attn_decode_workspace_bytes(B, H, Hkv, max_pages * page_size, d,
                                                 int(num_splits)))
    workspace, ws_bytes = _workspace(workspace, nbytes, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _check_buffer(out, q.shape, torch.bfloat16, q.device, "out")
    _check_buffer(lse, (B, H), torch.float32, q.device, "lse")
    with torch.cuda.device(q.device):
        _check(lib.attn_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                     _ptr(kv_lens), _ptr(out), _ptr(lse), B, H, Hkv, d,
                                     page_size, num_pages, max_pages, ctypes.c_float(scale),
                                     int(window), int(num_splits), _ptr(workspace),
                                     ctypes.c_size_t(ws_bytes), _stream(q.device)))
    return out, lse


def bwd_workspace_bytes(B, H, Hkv, Nq, Nk, d) -> int:
    return int(load_library().attn_bwd_workspace_bytes(B, H, Hkv, Nq, Nk, d))


def attn_bwd(q, k, v, o, lse, dout, scale=None, causal=False, window=0, dq=None, dk=None,
             dv=None, workspace=None):
    """Backward of attn_fwd (bf16): returns (dq like q, dk like k, dv like v).

    o and lse are attn_fwd's outputs for the same q, k, v, scale, causal and
    window; dout is the upstream gradient [B, H, Nq, d] bf16.
    """
    import torch
    B, H, Hkv, Nq, Nk, d = _fwd_checks(q, k, v)
    _require(q.dtype == torch.bfloat16, "the backward takes bfloat16")
    for t, name in ((o, "o"), (dout, "dout")):
        _require(t.shape == q.shape and t.dtype == q.dtype and t.device == q.device
                 and t.is_contiguous(), f"{name} must match q")
    _require(lse.shape == (B, H, Nq) and lse.dtype == torch.float32 and lse.device == q.device
             and lse.is_contiguous(), "lse must be fp32 [B, H, Nq]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, ref, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _check_buffer(t, ref.shape, ref.dtype, q.device, name)
    lib = load_library()
    nbytes = int(lib.attn_bwd_workspace_bytes(B, H, Hkv, Nq, Nk, d))
    workspace, ws_bytes = _workspace(workspace, nbytes, q.device)
    with torch.cuda.device(q.device):
        _check(lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                            _ptr(dk), _ptr(dv), B, H, Hkv, Nq, Nk, d, ctypes.c_float(scale),
                            int(bool(causal)), int(window), _ptr(workspace),
                            ctypes.c_size_t(ws_bytes), _stream(q.device)))
    return dq, dk, dv


def attn_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                    max_seqlen_k, scale=None, causal=False, window=0, dq=None, dk=None, dv=None,
                    workspace=None):
    """Backward of attn_fwd_varlen: returns (dq like q, dk like k, dv like v).

    q, o, dout [H, total_q, d] bf16; k, v [Hkv, total_k, d] bf16; lse
    [H, total_q] fp32 from attn_fwd_varlen with the same arguments.
    """
    import torch
    H, Hkv, total_q, total_k, d, ns = _varlen_checks(q, k, v, cu_seqlens_q, cu_seqlens_k)
    for t, name in ((o, "o"), (dout, "dout")):
        _require(t.shape == q.shape and t.dtype == q.dtype and t.device == q.device
                 and t.is_contiguous(), f"{name} must match q")
    _require(lse.shape == (H, total_q) and lse.dtype == torch.float32 and lse.device == q.device
             and lse.is_contiguous(), "lse must be fp32 [H, total_q]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, ref, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _check_buffer(t, ref.shape, ref.dtype, q.device, name)
    lib = load_library()
    nbytes = int(lib.attn_bwd_workspace_bytes(1, H, Hkv, total_q, total_k, d))
    workspace, ws_bytes = _workspace(workspace, nbytes, q.device)
    with torch.cuda.device(q.device):
        _check(lib.attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens_q),
                                   _ptr(cu_seqlens_k), ns, H, Hkv, total_q, total_k,
                                   int(max_seqlen_q), int(max_seqlen_k), d,
                                   ctypes.c_float(scale), int(bool(causal)), int(window),
                                   _ptr(workspace), ctypes.c_size_t(ws_bytes),
                                   _stream(q.device)))
    return dq, dk, dv


def calib_mfma(blocks: int, iters: int, sink):
    """Launch the bf16 matrix-core ceiling probe on the current stream."""
    lib = load_library()
    _check(lib.attn_calib_mfma(int(blocks), int(iters), _ptr(sink), _stream(sink.device)))
    return blocks * 4 * iters * 8 * 32768


def calib_read(buf, sink, blocks: int):
    """Launch the streaming-read ceiling probe over tensor `buf`."""
    lib = load_library()
    nbytes = buf.numel() * buf.element_size()
    _check(lib.attn_calib_read(_ptr(buf), ctypes.c_size_t(nbytes), _ptr(sink), int(blocks),
                               _stream(buf.device)))
    return nbytes
