"""Decode over a paged KV cache: HIP path against the oracle.

Parity on fragmented pools (shuffled physical pages, partial last pages,
empty and one-key sequences) for several page sizes; bit-identical results
to the contiguous mixed-length decode on the same keys; shared pages; table
entries past a sequence's length are never read; an entry outside the pool
reads as zeros without touching other memory. The paged decode workload at
full size is compared on every output in test_full_size.py.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import exact_io_aware_06_amd as mi
from helpers import check_lse, check_out, to64
from synth import inputs as S

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _gen(seed):
    return torch.Generator(device="cpu").manual_seed(seed)


def paged_case(lens, ps, H, Hkv, d, seed, extra_pages=0):
    table, npg = S.paged_block_table(seed, lens, ps)
    npg += extra_pages
    g = _gen(seed)
    q = torch.randn(len(lens), H, d, generator=g).to(torch.bfloat16)
    kp = torch.randn(npg, Hkv, ps, d, generator=g).to(torch.bfloat16)
    vp = torch.randn(npg, Hkv, ps, d, generator=g).to(torch.bfloat16)
    return q, kp, vp, table


def run_paged(q, kp, vp, table, lens, scale, window, splits):
    o, lse = mi.attn_decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV),
                                  torch.from_numpy(np.ascontiguousarray(table)).to(DEV),
                                  torch.as_tensor(lens, dtype=torch.int32).to(DEV),
                                  scale=scale, window=window, num_splits=splits)
    torch.cuda.synchronize()
    return o, lse


LENS = [0, 1, 15, 16, 17, 300, 1000]


@pytest.mark.parametrize("ps", [1, 16, 64, 256])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits,window", [(1, 0), (4, 0), (0, 0), (3, 50)])
def test_paged_parity(ps, d, splits, window):
    q, kp, vp, table = paged_case(LENS, ps, 8, 2, d, seed=ps + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = run_paged(q, kp, vp, table, LENS, scale, window, splits)
    o_ref, l_ref = oracle.decode_paged_ref(q, kp, vp, table, LENS, ps, scale, window)
    label = f"ps={ps} d={d} splits={splits} W={window}"
    check_out(to64(o), o_ref, label=label)
    check_lse(to64(lse), l_ref, label=label)


@pytest.mark.parametrize("H,Hkv", [(48, 1), (80, 2)])
def test_paged_many_heads_per_group(H, Hkv):
    """Groups of more than 32 query heads run in blocks of 32 over the same pages."""
    q, kp, vp, table = paged_case(LENS, 16, H, Hkv, 128, seed=H)
    o, lse = run_paged(q, kp, vp, table, LENS, 0.088, 0, 4)
    o_ref, l_ref = oracle.decode_paged_ref(q, kp, vp, table, LENS, 16, 0.088, 0)
    check_out(to64(o), o_ref, label=f"H={H} Hkv={Hkv}")
    check_lse(to64(lse), l_ref, label=f"H={H} Hkv={Hkv}")


@pytest.mark.parametrize("B", [256, 300])
def test_paged_large_batches(B):
    """Both ways of planning the balanced pieces (in the split work-groups up to 256
    sequences, by a plan kernel past that) over a paged cache."""
    r = np.random.default_rng(B + 1)
    lens = [int(x) for x in r.choice([0, 1, 16, 40, int(r.integers(0, 200))], B)]
    q, kp, vp, table = paged_case(lens, 16, 4, 2, 64, seed=B)
    o, lse = run_paged(q, kp, vp, table, lens, 0.125, 0, 2)
    o_ref, l_ref = oracle.decode_paged_ref(q, kp, vp, table, lens, 16, 0.125, 0)
    check_out(to64(o), o_ref, label=f"B={B}")
    check_lse(to64(lse), l_ref, label=f"B={B}")


@pytest.mark.parametrize("ps,splits", [(16, 1), (16, 8), (64, 5), (128, 16)])
def test_paged_matches_contiguous_decode(ps, splits):
    """Same keys, same chunks: identical to the contiguous mixed-length decode."""
    lens = [700, 1, 129, 1024, 513]
    q, kp, vp, table = paged_case(lens, ps, 32, 8, 128, seed=7)
    o1, l1 = run_paged(q, kp, vp, table, lens, 0.088, 0, splits)
    Nk = max(lens)
    kc = torch.zeros(len(lens), 8, Nk, 128, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    for b, n in enumerate(lens):
        kc[b, :, :n] = torch.from_numpy(oracle.gather_pages(kp, table, b, n, ps)).to(torch.bfloat16)
        vc[b, :, :n] = torch.from_numpy(oracle.gather_pages(vp, table, b, n, ps)).to(torch.bfloat16)
    o2, l2 = mi.attn_decode_varlen(q.to(DEV), kc.to(DEV), vc.to(DEV),
                                   torch.tensor(lens, dtype=torch.int32, device=DEV),
                                   scale=0.088, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_shared_pages():
    """Sequences naming the same physical pages (a shared prompt prefix)."""
    ps, d = 16, 128
    g = _gen(3)
    kp = torch.randn(12, 2, ps, d, generator=g).to(torch.bfloat16)
    vp = torch.randn(12, 2, ps, d, generator=g).to(torch.bfloat16)
    q = torch.randn(3, 8, d, generator=g).to(torch.bfloat16)
    table = np.array([[0, 1, 2, 3, 4], [0, 1, 2, 7, 8], [0, 1, 9, 10, 11]], dtype=np.int32)
    lens = [80, 70, 41]
    o, lse = run_paged(q, kp, vp, table, lens, 0.088, 0, 2)
    o_ref, l_ref = oracle.decode_paged_ref(q, kp, vp, table, lens, ps, 0.088, 0)
    check_out(to64(o), o_ref, label="shared pages")
    check_lse(to64(lse), l_ref, label="shared pages")


def test_paged_entries_past_length_are_never_read():
    lens = [33, 100, 5]
    ps = 16
    q, kp, vp, table = paged_case(lens, ps, 8, 2, 128, seed=4)
    wide = np.full((3, 10), -1, dtype=np.int32)
    wide[:, :table.shape[1]] = table
    o1, l1 = run_paged(q, kp, vp, wide, lens, 0.088, 0, 4)
    for b, n in enumerate(lens):
        wide[b, -(-n // ps):] = 1_000_000_000      # far outside the pool
    o2, l2 = run_paged(q, kp, vp, wide, lens, 0.088, 0, 4)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_entry_outside_pool_reads_zeros():
    """A bad page id inside a sequence: that page reads as zero keys and values."""
    lens = [48, 40]
    ps = 16
    q, kp, vp, table = paged_case(lens, ps, 8, 2, 128, seed=5)
    bad = table.copy()
    bad[0, 1] = 1 << 30
    o, lse = run_paged(q, kp, vp, bad, lens, 0.088, 0, 2)
    kz, vz = torch.cat([kp, torch.zeros_like(kp[:1])]), torch.cat([vp, torch.zeros_like(vp[:1])])
    zero_page = bad.copy()
    zero_page[0, 1] = kp.shape[0]                 # an explicit all-zero page
    o_ref, l_ref = oracle.decode_paged_ref(q, kz, vz, zero_page, lens, ps, 0.088, 0)
    check_out(to64(o), o_ref, label="zero page")
    check_lse(to64(lse), l_ref, label="zero page")
