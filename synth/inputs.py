"""Workload shapes and seeded N(0,1) tensors for the attention path.

Every tensor is drawn one batch index at a time from its own seeded torch
generator, so any batch slice can be rebuilt alone (the decode cache at full
size is 8.6 GB of bf16; rebuilding one sequence of it is 134 MB).

Generation recipe, for tensor ``tid`` (q=0, k=1, v=2), batch index ``b``:

* generator seeded with ``seed_key(seed, tid, b)`` on the requested device;
* ``torch.randn`` in float32;
* optional multiply by a float32 constant (the sharpened workload);
* one round-to-nearest-even cast to the storage dtype (bf16 or fp32).

The same seed on the same device type always yields the same bits. CPU and
GPU generators are different streams: a test draws on one device and copies
the tensors it needs to the other.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

TID_Q, TID_K, TID_V = 0, 1, 2


def seed_key(seed: int, tid: int, b: int) -> int:
    """Generator seed for tensor ``tid``, batch index ``b`` of run ``seed``."""
    return int(seed) * 10_000_000 + int(tid) * 100_000 + int(b)


def _dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def gen_normal(shape, seed: int, tid: int, b: int, dtype: str = "bf16",
               mult: float = 1.0, device="cpu") -> torch.Tensor:
    """One batch slice: N(0,1) float32, times ``mult`` in float32, then RNE cast."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed_key(seed, tid, b))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=dev)
    if mult != 1.0:
        x.mul_(float(np.float32(mult)))
    return x.to(_dtype(dtype))


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    H: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str          # "bf16" or "f32"
    causal: int
    window: int
    scale: float        # the value handed to the kernel (float32-representable)
    qk_mult: float = 1.0  # applied to Q and K before the cast (sharpened logits)
    note: str = ""

    def with_(self, **kw) -> "PrefillConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return PrefillConfig(**d)


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    H: int
    Hkv: int
    Nk: int
    d: int
    splits: int
    scale: float
    window: int = 0
    dtype: str = "bf16"
    note: str = ""

    def with_(self, **kw) -> "DecodeConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return DecodeConfig(**d)


def _f32(x: float) -> float:
    return float(np.float32(x))


# The five workloads. Shapes follow the contexts the pages discuss (2k-8k
# training contexts, 32k documents, KV-cache decode); values are i.i.d. N(0,1).
CONFIGS = {
    "f32_n256_d64": PrefillConfig("f32_n256_d64", 1, 1, 1, 256, 256, 64, "f32", 0, 0, _f32(1 / 8),
                        note="single head, non-causal, fp32"),
    "causal_b4_h16_n2048_d64": PrefillConfig("causal_b4_h16_n2048_d64", 4, 16, 16, 2048, 2048, 64, "bf16", 1, 0, _f32(1 / 8),
                        note="causal self-attention prefill"),
    # Q and K are each multiplied by 3 * d^-1/4 before the bf16 cast, which folds
    # the 1/sqrt(d) into the inputs and sharpens the logits threefold; the kernel
    # scale is therefore 1.0.
    "causal_gqa_n8192_d128": PrefillConfig("causal_gqa_n8192_d128", 1, 32, 8, 8192, 8192, 128, "bf16", 1, 0, 1.0,
                        qk_mult=3.0 * 128 ** -0.25,
                        note="causal GQA prefill, sharpened logits"),
    "window4096_gqa_n32768_d128": PrefillConfig("window4096_gqa_n32768_d128", 1, 32, 8, 32768, 32768, 128, "bf16", 1, 4096,
                        _f32(1 / math.sqrt(128)),
                        note="causal sliding-window GQA prefill"),
    "decode_b64_nk32768_d128": DecodeConfig("decode_b64_nk32768_d128", 64, 32, 8, 32768, 128, 16, _f32(1 / math.sqrt(128)),
                       note="split-K decode over a 32k KV cache"),
}


def prefill_inputs(cfg: PrefillConfig, seed: int, device="cpu", batches=None):
    """(q, k, v) for a prefill config: q [B,H,Nq,d], k/v [B,Hkv,Nk,d].

    ``batches`` restricts generation to a list of batch indices (the result
    then has len(batches) rows in dim 0).
    """
    bs = range(cfg.B) if batches is None else list(batches)
    qs, ks, vs = [], [], []
    for b in bs:
        qs.append(gen_normal((cfg.H, cfg.Nq, cfg.d), seed, TID_Q, b, cfg.dtype,
                             cfg.qk_mult, device))
        ks.append(gen_normal((cfg.Hkv, cfg.Nk, cfg.d), seed, TID_K, b, cfg.dtype,
                             cfg.qk_mult, device))
        vs.append(gen_normal((cfg.Hkv, cfg.Nk, cfg.d), seed, TID_V, b, cfg.dtype,
                             1.0, device))
    return torch.stack(qs), torch.stack(ks), torch.stack(vs)


def decode_inputs(cfg: DecodeConfig, seed: int, device="cpu", batches=None):
    """(q, k_cache, v_cache) for decode: q [B,H,d], caches [B,Hkv,Nk,d].

    The caches are filled in place one sequence at a time so peak host memory
    stays at one sequence of float32 on top of the bf16 result.
    """
    bs = range(cfg.B) if batches is None else list(batches)
    n = len(bs)
    dt = _dtype(cfg.dtype)
    q = torch.empty((n, cfg.H, cfg.d), dtype=dt, device=device)
    kc = torch.empty((n, cfg.Hkv, cfg.Nk, cfg.d), dtype=dt, device=device)
    vc = torch.empty_like(kc)
    for i, b in enumerate(bs):
        q[i] = gen_normal((cfg.H, cfg.d), seed, TID_Q, b, cfg.dtype, 1.0, device)
        kc[i] = gen_normal((cfg.Hkv, cfg.Nk, cfg.d), seed, TID_K, b, cfg.dtype, 1.0, device)
        vc[i] = gen_normal((cfg.Hkv, cfg.Nk, cfg.d), seed, TID_V, b, cfg.dtype, 1.0, device)
    return q, kc, vc


# ---------------------------------------------------------------------------
# Packed variable-length sequences and per-sequence KV-cache lengths.
#
# Lengths come from numpy generators seeded with seed_key(seed, TID_LEN, unit),
# one per training context (packed prefill) or one per batch (decode), so the
# length mix is fixed by the seed alone.

TID_LEN = 3


def packed_lengths(seed: int, contexts: int, context_len: int, min_len: int,
                   max_len: int) -> list:
    """Document lengths filling ``contexts`` training contexts of ``context_len`` tokens.

    Each context is filled with documents whose lengths are drawn
    log-uniformly in [min_len, max_len] (rounded down to an integer); the
    document that would run past the end of the context is cut there, so no
    document spans two contexts and every context holds exactly
    ``context_len`` tokens.
    """
    out = []
    for c in range(contexts):
        rng = np.random.default_rng(seed_key(seed, TID_LEN, c))
        left = context_len
        while left > 0:
            n = int(math.exp(rng.uniform(math.log(min_len), math.log(max_len + 1))))
            n = max(1, min(n, max_len, left))
            out.append(n)
            left -= n
    return out


def cu_seqlens(lengths) -> np.ndarray:
    """int32 offsets [len(lengths) + 1]: 0, then the running totals."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu.astype(np.int32)


def kv_lengths(seed: int, B: int, Nk: int, lo: int = 1) -> np.ndarray:
    """int32 [B]: per-sequence cache lengths, uniform integers in [lo, Nk]."""
    rng = np.random.default_rng(seed_key(seed, TID_LEN, 0))
    return rng.integers(lo, Nk + 1, size=B).astype(np.int32)


def skewed_kv_lengths(B: int, Nk: int, every: int = 8, short: int = 512) -> np.ndarray:
    """int32 [B]: a serving batch dominated by a few long contexts: every
    `every`-th sequence holds all Nk keys, the others `short` keys."""
    lens = np.full(B, min(short, Nk), dtype=np.int32)
    lens[::every] = Nk
    return lens


@dataclass(frozen=True)
class PackedConfig:
    name: str
    H: int
    Hkv: int
    d: int
    contexts: int       # training contexts, each packed with documents
    context_len: int    # tokens per context
    min_len: int        # document length range (log-uniform)
    max_len: int
    causal: int
    window: int
    scale: float
    dtype: str = "bf16"
    note: str = ""

    def with_(self, **kw) -> "PackedConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return PackedConfig(**d)

    def lengths(self, seed: int) -> list:
        return packed_lengths(seed, self.contexts, self.context_len, self.min_len,
                              self.max_len)


# Packed prefill: four 8k training contexts ("What Lost, and Why": 2k-8k
# training contexts) each filled with documents of log-uniform length in
# [64, 8192], causal, the GQA head shape of the prefill workloads.
PACKED = {
    "packed_24docs_4x8192_d128": PackedConfig("packed_24docs_4x8192_d128", 32, 8, 128, 4, 8192, 64, 8192, 1, 0,
                       _f32(1 / math.sqrt(128)),
                       note="packed causal GQA prefill, 4 x 8k contexts, log-uniform documents"),
}

# Decode over caches of mixed length: the decode workload's shapes with each
# sequence holding a uniform random number of keys in [1, 32768].
DECODE_KVLENS = CONFIGS["decode_b64_nk32768_d128"].with_(name="decode_kvlens_b64_nk32768_d128", note="split-K decode, per-sequence cache lengths")


def packed_inputs(cfg: PackedConfig, total_q: int, total_k: int, seed: int, device="cpu"):
    """(q, k, v) packed: q [H, total_q, d], k/v [Hkv, total_k, d]."""
    q = gen_normal((cfg.H, total_q, cfg.d), seed, TID_Q, 0, cfg.dtype, 1.0, device)
    k = gen_normal((cfg.Hkv, total_k, cfg.d), seed, TID_K, 0, cfg.dtype, 1.0, device)
    v = gen_normal((cfg.Hkv, total_k, cfg.d), seed, TID_V, 0, cfg.dtype, 1.0, device)
    return q, k, v


def paged_block_table(seed: int, kv_lens, page_size: int, max_pages: int | None = None):
    """(block_table int32 [B, max_pages], num_pages) for a fragmented page pool.

    Sequence b gets ceil(kv_lens[b] / page_size) pages. The physical page ids
    are a seeded random permutation of 0 .. num_pages - 1, so neighbouring
    pages of a sequence are scattered over the pool; unused entries are -1.
    """
    lens = np.asarray(kv_lens, dtype=np.int64)
    need = -(-lens // page_size)
    num_pages = int(need.sum())
    width = int(need.max(initial=0)) if max_pages is None else int(max_pages)
    rng = np.random.default_rng(seed_key(seed, TID_LEN, 1))
    perm = rng.permutation(num_pages)
    table = np.full((lens.size, max(width, 1)), -1, dtype=np.int32)
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[at:at + n]
        at += n
    return table, num_pages


# Paged decode: the mixed-length decode workload stored in 16-key pages
# scattered over one pool.
PAGED = {"page_size": 16, "decode": CONFIGS["decode_b64_nk32768_d128"].with_(name="decode_paged16_b64_nk32768_d128",
                                                         note="split-K decode over a paged cache")}


def paged_inputs(cfg: DecodeConfig, num_pages: int, page_size: int, seed: int, device="cpu"):
    """(q [B,H,d], k_pages, v_pages [num_pages, Hkv, page_size, d]) for paged decode."""
    q = gen_normal((cfg.B, cfg.H, cfg.d), seed, TID_Q, 0, cfg.dtype, 1.0, device)
    k = gen_normal((num_pages, cfg.Hkv, page_size, cfg.d), seed, TID_K, 0, cfg.dtype, 1.0, device)
    v = gen_normal((num_pages, cfg.Hkv, page_size, cfg.d), seed, TID_V, 0, cfg.dtype, 1.0, device)
    return q, k, v


# ---------------------------------------------------------------------------
# FP8 (OCP e4m3fn) inputs with one fp32 descale per tensor.

FP8_MAX = 448.0


def quantize_fp8(x: torch.Tensor):
    """(x8 float8_e4m3fn, descale float) with x ~= x8 * descale.

    descale = amax / 448 in fp32, so the largest |x| maps to the largest
    finite e4m3fn value; every element is rounded to nearest even once.
    """
    amax = float(x.abs().max()) if x.numel() else 0.0
    descale = float(np.float32(amax / FP8_MAX)) if amax > 0 else 1.0
    x8 = (x.to(torch.float32) / descale).to(torch.float8_e4m3fn)
    return x8, descale


def fp8_prefill_inputs(cfg: PrefillConfig, seed: int, device="cpu"):
    """(q8, k8, v, q_descale, k_descale): the prefill config's Q and K drawn as
    for bf16 (fp32 randn times qk_mult) and quantized per tensor to e4m3fn; V bf16."""
    qs, ks, vs = [], [], []
    for b in range(cfg.B):
        qs.append(gen_normal((cfg.H, cfg.Nq, cfg.d), seed, TID_Q, b, "f32", cfg.qk_mult, device))
        ks.append(gen_normal((cfg.Hkv, cfg.Nk, cfg.d), seed, TID_K, b, "f32", cfg.qk_mult, device))
        vs.append(gen_normal((cfg.Hkv, cfg.Nk, cfg.d), seed, TID_V, b, "bf16", 1.0, device))
    q8, qd = quantize_fp8(torch.stack(qs))
    k8, kd = quantize_fp8(torch.stack(ks))
    return q8, k8, torch.stack(vs), qd, kd
