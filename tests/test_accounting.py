"""Work/traffic accounting and the tile enumerator, pinned to the pages' figures
and to brute-force counts over the visibility mask."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle.attention import visible_mask
from exact_io_aware_06_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def figures():
    with open(GOLDEN) as f:
        return {e["id"]: e["value"] for e in json.load(f)["figures"]}


def test_page_figures():
    fig = figures()
    # 32k vs 1k tokens: 1,024x the attention operations (full attention).
    assert acc.dense_attention_ops(32 * 1024, 128) // acc.dense_attention_ops(1024, 128) \
        == fig["ops_32k_vs_1k"]
    assert acc.prefill_flops(1, 1, 32768, 32768, 128, False, 0) \
        // acc.prefill_flops(1, 1, 1024, 1024, 128, False, 0) == fig["ops_32k_vs_1k"]
    # 2K -> 128K: 4,096x compute and memory.
    assert acc.prefill_flops(1, 1, 131072, 131072, 64, False, 0) \
        // acc.prefill_flops(1, 1, 2048, 2048, 64, False, 0) == fig["cost_2k_to_128k"]
    assert acc.score_matrix_bytes(131072) // acc.score_matrix_bytes(2048) == fig["cost_2k_to_128k"]
    # doubling the context quadruples the work
    assert acc.dense_attention_ops(4096) == fig["doubling_factor"] * acc.dense_attention_ops(2048)
    # one head, 64k tokens, FP32 scores: ~16 GB (2^34 bytes = 16 GiB)
    assert acc.score_matrix_bytes(65536, 4) / 2 ** 30 == fig["score_bytes_64k_fp32_gb"]
    # n = 1000 -> 1,000,000 entries
    assert acc.score_matrix_bytes(1000, 1) == fig["entries_n1000"]
    assert acc.visible_pairs(1000, 1000, False, 0) == fig["entries_n1000"]
    # 100,000 tokens -> 10 billion interactions per head
    assert acc.visible_pairs(100_000, 100_000, False, 0) == fig["interactions_n100k"]
    # full vs local window, n = 100000, w = 512: n / w ~ 195
    assert round(100_000 / 512) == fig["full_vs_window_n100k_w512"]
    full = acc.dense_attention_ops(100_000)
    assert round(full / (100_000 * 512)) == fig["full_vs_window_n100k_w512"]


@pytest.mark.parametrize("Nq,Nk,causal,window", [
    (1, 1, 1, 0), (33, 33, 1, 0), (33, 33, 0, 0), (33, 33, 1, 5), (33, 33, 0, 5),
    (20, 50, 1, 0), (50, 20, 1, 0), (50, 20, 1, 3), (50, 20, 0, 3), (7, 300, 1, 64),
])
def test_visible_pairs_equals_mask_count(Nq, Nk, causal, window):
    assert acc.visible_pairs(Nq, Nk, causal, window) == \
        int(visible_mask(Nq, Nk, causal, window).sum())


def test_visible_pairs_closed_forms():
    # causal: N(N+1)/2 per head
    assert acc.visible_pairs(8192, 8192, True, 0) == 8192 * 8193 // 2
    # causal window W: rows see min(p+1, W+1) keys
    N, W = 32768, 4096
    expect = sum(min(p + 1, W + 1) for p in range(N))
    assert acc.visible_pairs(N, N, True, W) == expect == 125_859_840


def test_workload_totals():
    # causal GQA prefill at N=8192, d=128, 32 heads
    assert acc.prefill_flops(1, 32, 8192, 8192, 128, True, 0) == 549_822_922_752
    # split-K decode over a 32k cache, 64 sequences, 8 KV heads, d=128
    assert acc.decode_bytes(64, 32, 8, 32768, 128) == 8_590_991_360


def test_tile_enumerator_small_matches_mask():
    for (Nq, Nk, causal, window, BM, BN) in [(100, 100, 1, 0, 16, 8), (100, 130, 1, 20, 16, 32),
                                             (70, 70, 0, 9, 32, 16), (90, 40, 1, 0, 32, 16)]:
        need, full = oracle.tiles_needed(Nq, Nk, causal, window, BM, BN)
        vis = visible_mask(Nq, Nk, causal, window)
        for qt in range(need.shape[0]):
            for kt in range(need.shape[1]):
                blk = vis[qt * BM:(qt + 1) * BM, kt * BN:(kt + 1) * BN]
                assert need[qt, kt] == blk.any()
        assert not np.any(full & ~need)


@pytest.mark.slow
def test_tile_counts_sliding_window_workload():
    """Causal window 4096 at N=32768 with 128x64 tiles: 15,840 of 65,792 key tiles."""
    need, full = oracle.tiles_needed(32768, 32768, True, 4096, 128, 64)
    assert int(need.sum()) == 15_840
    need_c, _ = oracle.tiles_needed(32768, 32768, True, 0, 128, 64)
    assert int(need_c.sum()) == 256 * 257
    assert int((need & ~full).sum()) == 960
