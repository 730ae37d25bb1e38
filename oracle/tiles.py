"""Which score-matrix blocks hold any visible (query, key) pair.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Straight from the visibility definition: a (query-tile, key-tile) block must
be computed iff at least one pair in it is visible, and needs no mask iff
every pair in it is visible. Tiled kernels that skip whole blocks for causal
and sliding-window masks ("Attention Research", section 4: irregular sparsity
maps badly to matrix units, so whole blocks are skipped instead) must visit
exactly the "needed" set.
"""

from __future__ import annotations

import numpy as np

from .attention import visible_mask


def tiles_needed(Nq: int, Nk: int, causal: bool, window: int, BM: int, BN: int):
    """Returns (needed [nqt, nkt] bool, full [nqt, nkt] bool) by brute force.

    A block that runs past Nq or Nk is "full" only if its in-range part is all
    visible and it does not run past Nk (keys past the end must be masked).
    """
    nqt = -(-Nq // BM)
    nkt = -(-Nk // BN)
    needed = np.zeros((nqt, nkt), dtype=bool)
    full = np.zeros((nqt, nkt), dtype=bool)
    for qt in range(nqt):
        rows = np.arange(qt * BM, min(Nq, qt * BM + BM))
        vis = visible_mask(Nq, Nk, causal, window, rows)
        for kt in range(nkt):
            blk = vis[:, kt * BN:min(Nk, kt * BN + BN)]
            needed[qt, kt] = blk.any()
            full[qt, kt] = blk.all() and (kt * BN + BN <= Nk)
    return needed, full
