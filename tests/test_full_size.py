"""Parity at the full workload sizes, against the fp64 oracle, seeds 0, 1 and 2.

The method's claim is the same output as the plain definition, up to
rounding ("Chapter 3.1 - The Cost of Attention", section 5; grasp.study
efficient-attention lesson, "Online Softmax"). These tests compare every
output element of the workloads the oracle can evaluate in seconds, with the
max-abs and mean-abs bounds taken over the whole tensor:

* causal GQA prefill, B1 H32 Hkv8 N8192 d128 (sharpened logits): every O and
  LSE element, all 32 heads;
* split-K decode, B64 H32 Hkv8 Nk32768 d128, 16 splits: every sequence and
  head, one sequence of the cache at a time on the host;
* packed documents (four 8k contexts, H32 Hkv8): every row of every head;
* decode with per-sequence lengths, the same over 16-key pages, and a skewed
  batch (every eighth sequence full, the rest 512 keys): every sequence and head.

The causal sliding-window prefill over 32768 tokens (window 4096) would need
the full 32768 x 32768 score matrix per head in the oracle, so it is compared
on dense row blocks of every head: the first and last two query tiles, the
rows around the window's edge (4095-4225), every 512th row and a seeded 2 %
of all rows.

The causal context sweep (B1 H32 Hkv8 d128, N(0,1) inputs, scale 1/sqrt(d),
N = 1k ... 128k) is compared on every output up to 8k tokens, and from 16k
on, where the oracle's full score matrix grows to 34-550 GB per run, on dense
row blocks of all 32 heads: the first and last query tiles, four seeded
blocks of 128 consecutive rows and every (N/64)-th row, each row against all
N keys.

The kernels run exactly as in the benchmark (same entry points, same split
count and tile configuration).
"""

import sys
import time

import numpy as np
import pytest
import torch

import oracle
import synth
import exact_io_aware_06_amd as mi
from helpers import check_lse, check_out, to64
from synth import inputs as S

pytestmark = pytest.mark.gpu

DEV = "cuda"
SEEDS = [0, 1, 2]


def note(msg):
    print(f"[full-size] {msg}", file=sys.stderr, flush=True)


def compare(o_gpu, o_ref, l_gpu, l_ref, label):
    mx, mean = check_out(o_gpu, o_ref, bf16=True, label=label)
    lerr = check_lse(l_gpu, l_ref, label=label)
    note(f"{label}: O max-abs {mx:.3e} mean-abs {mean:.3e}, LSE max-abs {lerr:.3e}")


@pytest.mark.parametrize("seed", SEEDS)
def test_causal_gqa_n8192_every_output(seed):
    c = synth.CONFIGS["causal_gqa_n8192_d128"]
    note(f"{c.name} seed {seed}: GPU")
    q, k, v = synth.prefill_inputs(c, seed)
    o, lse = mi.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=c.scale, causal=c.causal,
                         window=c.window)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    o_ref, l_ref = oracle.attention_ref(q, k, v, c.scale, c.causal, c.window)
    note(f"{c.name} seed {seed}: oracle {time.perf_counter() - t0:.1f} s")
    compare(to64(o), o_ref, to64(lse), l_ref, f"{c.name} seed {seed}")


def window_rows(N, W, seed):
    rng = np.random.default_rng(1000 + seed)
    rows = set(range(0, 256)) | set(range(N - 256, N))
    rows |= set(range(W - 1, W + 130))          # the window edge, 4095 .. 4225
    rows |= set(range(0, N, 512))
    rows |= set(rng.choice(N, size=N // 50, replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("seed", SEEDS)
def test_sliding_window_n32768_dense_rows(seed):
    c = synth.CONFIGS["window4096_gqa_n32768_d128"]
    note(f"{c.name} seed {seed}: GPU")
    q, k, v = synth.prefill_inputs(c, seed)
    o, lse = mi.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=c.scale, causal=c.causal,
                         window=c.window)
    torch.cuda.synchronize()
    og, lg = o.cpu(), lse.cpu()
    assert torch.isfinite(og.float()).all() and torch.isfinite(lg).all()
    rows = window_rows(c.Nq, c.window, seed)
    t0 = time.perf_counter()
    o_ref = np.empty((c.H, rows.size, c.d))
    l_ref = np.empty((c.H, rows.size))
    for h in range(c.H):
        o_ref[h], l_ref[h] = oracle.attention_rows_ref(q, k, v, c.scale, c.causal, c.window,
                                                       0, h, rows)
    note(f"{c.name} seed {seed}: oracle on {rows.size} rows x {c.H} heads "
         f"{time.perf_counter() - t0:.1f} s")
    compare(to64(og[0][:, rows]), o_ref, to64(lg[0][:, rows]), l_ref, f"{c.name} seed {seed}")


def decode_all_sequences(o, lse, ref_fn, B, label):
    og, lg = to64(o), to64(lse)
    o_ref = np.empty_like(og)
    l_ref = np.empty_like(lg)
    t0 = time.perf_counter()
    for b in range(B):
        o_ref[b], l_ref[b] = ref_fn(b)
    note(f"{label}: oracle {time.perf_counter() - t0:.1f} s")
    compare(og, o_ref, lg, l_ref, label)


@pytest.mark.parametrize("seed", SEEDS)
def test_decode_b64_nk32768_every_output(seed):
    c = synth.CONFIGS["decode_b64_nk32768_d128"]
    note(f"{c.name} seed {seed}: GPU")
    q, kc, vc = synth.decode_inputs(c, seed=seed, device=DEV)
    o, lse = mi.attn_decode(q, kc, vc, scale=c.scale, num_splits=c.splits)
    torch.cuda.synchronize()
    heads = list(range(c.H))

    def ref(b):
        return oracle.decode_rows_ref(q[b:b + 1].cpu(), kc[b:b + 1].cpu(), vc[b:b + 1].cpu(),
                                      c.scale, c.window, 0, heads)

    decode_all_sequences(o, lse, ref, c.B, f"{c.name} seed {seed}")
    del kc, vc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed", SEEDS)
def test_packed_documents_every_output(seed):
    cfg = S.PACKED["packed_24docs_4x8192_d128"]
    lens = cfg.lengths(seed)
    cu = S.cu_seqlens(lens)
    total = int(cu[-1])
    note(f"{cfg.name} seed {seed}: {len(lens)} documents, GPU")
    q, k, v = S.packed_inputs(cfg, total, total, seed=seed)
    cu_dev = torch.from_numpy(cu).to(DEV)
    o, lse = mi.attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu_dev, cu_dev, max(lens),
                                scale=cfg.scale, causal=cfg.causal, window=cfg.window)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    o_ref, l_ref = oracle.attention_varlen_ref(q, k, v, cu, cu, cfg.scale, cfg.causal,
                                               cfg.window)
    note(f"{cfg.name} seed {seed}: oracle {time.perf_counter() - t0:.1f} s")
    compare(to64(o), o_ref, to64(lse), l_ref, f"{cfg.name} seed {seed}")


@pytest.mark.parametrize("seed", SEEDS)
def test_decode_kvlens_every_output(seed):
    c = S.DECODE_KVLENS
    lens = S.kv_lengths(seed, c.B, c.Nk)
    note(f"{c.name} seed {seed}: {int(lens.sum())} keys, GPU")
    q, kc, vc = S.decode_inputs(c, seed, device=DEV)
    o, lse = mi.attn_decode_varlen(q, kc, vc, torch.from_numpy(lens).to(DEV), scale=c.scale,
                                   num_splits=c.splits)
    torch.cuda.synchronize()
    heads = list(range(c.H))

    def ref(b):
        n = int(lens[b])
        return oracle.decode_kvlens_rows_ref(q[b:b + 1].cpu(), kc[b:b + 1, :, :n].cpu(),
                                             vc[b:b + 1, :, :n].cpu(), [n], c.scale, c.window,
                                             0, heads)

    decode_all_sequences(o, lse, ref, c.B, f"{c.name} seed {seed}")
    del kc, vc
    torch.cuda.empty_cache()


def test_decode_skewed_lengths_every_output():
    """The bench's skewed batch: every eighth sequence holds all 32768 keys, the rest 512;
    balanced pieces spread each long sequence over many work-groups."""
    c = S.DECODE_KVLENS
    lens = S.skewed_kv_lengths(c.B, c.Nk)
    note(f"skewed decode: {int(lens.sum())} keys, GPU")
    q, kc, vc = S.decode_inputs(c, 0, device=DEV)
    o, lse = mi.attn_decode_varlen(q, kc, vc, torch.from_numpy(lens).to(DEV), scale=c.scale,
                                   num_splits=c.splits)
    torch.cuda.synchronize()
    heads = list(range(c.H))

    def ref(b):
        n = int(lens[b])
        return oracle.decode_kvlens_rows_ref(q[b:b + 1].cpu(), kc[b:b + 1, :, :n].cpu(),
                                             vc[b:b + 1, :, :n].cpu(), [n], c.scale, c.window,
                                             0, heads)

    decode_all_sequences(o, lse, ref, c.B, "skewed decode")
    del kc, vc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed", SEEDS)
def test_decode_paged_every_output(seed):
    c = S.PAGED["decode"]
    ps = S.PAGED["page_size"]
    lens = S.kv_lengths(seed, c.B, c.Nk)
    table, npg = S.paged_block_table(seed, lens, ps)
    note(f"{c.name} seed {seed}: {npg} pages, GPU")
    q, kp, vp = S.paged_inputs(c, npg, ps, seed, device=DEV)
    o, lse = mi.attn_decode_paged(q, kp, vp, torch.from_numpy(table).to(DEV),
                                  torch.from_numpy(lens).to(DEV), scale=c.scale,
                                  num_splits=c.splits)
    torch.cuda.synchronize()
    qh = q.cpu()

    def ref(b):
        n = int(lens[b])
        used = table[b:b + 1, :-(-n // ps)]
        uniq = np.unique(used)
        pages = torch.from_numpy(uniq).to(DEV)
        local = np.searchsorted(uniq, used).astype(np.int32)    # page ids within the copy
        ob, lb = oracle.decode_paged_ref(qh[b:b + 1], kp[pages].cpu(), vp[pages].cpu(), local,
                                         [n], ps, c.scale, c.window)
        return ob[0], lb[0]

    decode_all_sequences(o, lse, ref, c.B, f"{c.name} seed {seed}")
    del kp, vp
    torch.cuda.empty_cache()


SWEEP = [1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072]


def sweep_rows(N, seed):
    rng = np.random.default_rng(2000 + N + seed)
    rows = set(range(0, 128)) | set(range(N - 128, N)) | set(range(0, N, N // 64))
    for start in rng.choice(N // 128, size=4, replace=False):
        rows |= set(range(int(start) * 128, int(start) * 128 + 128))
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("N", SWEEP)
def test_causal_context_sweep(N):
    c = synth.CONFIGS["window4096_gqa_n32768_d128"].with_(name=f"causal{N}", Nq=N, Nk=N,
                                                          window=0)
    note(f"{c.name}: GPU")
    q, k, v = synth.prefill_inputs(c, 0, device=DEV)
    o, lse = mi.attn_fwd(q, k, v, scale=c.scale, causal=c.causal, window=c.window)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if N <= 8192:
        qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
        o_ref, l_ref = oracle.attention_ref(qh, kh, vh, c.scale, c.causal, c.window)
        og, lg = to64(o), to64(lse)
        what = "every output"
    else:
        rows = sweep_rows(N, 0)
        o_ref = np.empty((c.H, rows.size, c.d))
        l_ref = np.empty((c.H, rows.size))
        kh, vh = k.cpu(), v.cpu()
        for h in range(c.H):
            o_ref[h], l_ref[h] = oracle.attention_rows_ref(q, kh, vh, c.scale, c.causal,
                                                           c.window, 0, h, rows)
        og, lg = to64(o[0][:, rows]), to64(lse[0][:, rows])
        what = f"{rows.size} rows x {c.H} heads"
    note(f"{c.name}: oracle on {what} {time.perf_counter() - t0:.1f} s")
    compare(og, o_ref, lg, l_ref, f"{c.name} ({what})")
    del q, k, v, o, lse
    torch.cuda.empty_cache()


# The longest key range the C ABI takes for one head: the K / V rows of one
# head are addressed through 32-bit buffer offsets, so Nk * d * 4 must stay
# below 2^32 (8,388,607 keys at d = 128; one more is refused, tests/test_abi.py).
NK_MAX_D128 = 0xFFFFFFFF // (128 * 4)
MAX_ROWS = np.array([0, 1, 63, 64, 127, 128, 129, 190, 199])


@pytest.mark.parametrize("causal,window", [(0, 0), (1, 5000)])
def test_longest_key_range(causal, window):
    """Two query heads of one K/V head against 8,388,607 keys (Nq = 200, so the
    second query tile is ragged). Non-causal, every row sees every key; causal
    with a window, the rows sit at the far end of the keys, so the tiles
    visited are the last ones and their buffer offsets the largest. Sampled
    rows of both heads (first and last rows of each query tile) against the
    oracle, each row against all keys."""
    c = synth.CONFIGS["window4096_gqa_n32768_d128"].with_(
        name=f"max_keys_c{causal}_w{window}", B=1, H=2, Hkv=1, Nq=200, Nk=NK_MAX_D128,
        causal=causal, window=window)
    note(f"{c.name}: GPU, Nk = {c.Nk}")
    q, k, v = synth.prefill_inputs(c, 0, device=DEV)
    o, lse = mi.attn_fwd(q, k, v, scale=c.scale, causal=causal, window=window)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    qh = q.cpu()
    # K / V widened once on the host (8.6 GB each), shared by both heads' rows
    kh = k.cpu().to(torch.float64).numpy()
    vh = v.cpu().to(torch.float64).numpy()
    del k, v
    torch.cuda.empty_cache()
    o_ref = np.empty((c.H, MAX_ROWS.size, c.d))
    l_ref = np.empty((c.H, MAX_ROWS.size))
    for h in range(c.H):
        o_ref[h], l_ref[h] = oracle.attention_rows_ref(qh, kh, vh, c.scale, causal, window, 0,
                                                       h, MAX_ROWS)
    note(f"{c.name}: oracle on {MAX_ROWS.size} rows x {c.H} heads {time.perf_counter() - t0:.1f} s")
    compare(to64(o[0][:, MAX_ROWS]), o_ref, to64(lse[0][:, MAX_ROWS]), l_ref, c.name)
    del q, o, lse, kh, vh
    torch.cuda.empty_cache()


def test_decode_cache_past_4_gib():
    """Decode over caches larger than 4 GiB per tensor (three sequences of
    6,000,007 keys, H8 Hkv1 d128: 4.6 GB each for K and V), so the third
    sequence's rows sit at byte offsets beyond 2^32; the library's split
    count. Every sequence and head against the oracle."""
    c = synth.CONFIGS["decode_b64_nk32768_d128"].with_(name="decode_past_4gib", B=3, H=8, Hkv=1,
                                                       Nk=6_000_007, splits=0)
    assert c.Nk * c.d * 2 * (c.B - 1) < 2 ** 32 < c.Nk * c.d * 2 * c.B
    note(f"{c.name}: GPU")
    q, kc, vc = synth.decode_inputs(c, seed=0, device=DEV)
    o, lse = mi.attn_decode(q, kc, vc, scale=c.scale, num_splits=0)
    torch.cuda.synchronize()
    heads = list(range(c.H))

    def ref(b):
        return oracle.decode_rows_ref(q[b:b + 1].cpu(), kc[b:b + 1].cpu(), vc[b:b + 1].cpu(),
                                      c.scale, c.window, 0, heads)

    decode_all_sequences(o, lse, ref, c.B, c.name)
    del kc, vc
    torch.cuda.empty_cache()
