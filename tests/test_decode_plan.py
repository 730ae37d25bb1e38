"""The work plan of split-K decode with per-sequence lengths, as a model on the host.

With per-sequence cache lengths the decode does not cut each sequence into S
equal chunks. It lays the visible keys of all sequences end to end in tiles of
128 keys, each sequence that has keys preceded by PIECE virtual tiles (for
what a piece costs beyond its tiles), and hands each of its W work-groups per
KV head (at most B * S; the launch caps W at one round of the work-groups the
device holds at once) an equal run of these units; a run that crosses a
sequence boundary yields one partial result per sequence it touches (empty
when the run holds only that sequence's virtual tiles), and the partial of
(work-group w, sequence b) is stored as partial w + b. The merge finds a
sequence's partials from the running unit counts alone.

This test restates that plan in plain Python and checks the properties the
kernels rely on, over random batches (empty sequences, one-key sequences,
windows, ragged lengths, more work-groups than tiles):

* every visible key of every sequence is covered exactly once, in order;
* the partial index w + b is unique (if b1 < b2, every tile of b1 precedes
  every tile of b2, so w1 <= w2), and below B (S + 1);
* the partials the merge reads for a sequence are exactly the ones written.

The GPU tests (test_varlen.py, test_paged.py, test_random_shapes.py,
test_full_size.py) check the kernels' results against the oracle; this one
pins the indexing argument itself.
"""

import random

import pytest

TILE = 128
PIECE = 1  # virtual tiles per sequence with keys


def visible(n, Nk, window):
    """Keys [vis, n) that the query at position n - 1 sees."""
    n = min(max(n, 0), Nk)
    vis = max(0, n - 1 - window) if window > 0 else 0
    return vis, n


def plan(lens, Nk, window, W):
    """Running tile counts T[0..B], tiles per work-group, first sequence of each work-group."""
    T = [0]
    for n in lens:
        vis, hi = visible(n, Nk, window)
        t = (hi - vis + TILE - 1) // TILE
        T.append(T[-1] + (t + PIECE if t > 0 else 0))
    total = T[-1]
    budget = max(1, -(-total // W))
    first = {}
    for b in range(len(lens)):
        w = -(-T[b] // budget)
        while w * budget < T[b + 1]:
            first[w] = b
            w += 1
    return T, budget, first


def run_plan(lens, Nk, window, S, W=None):
    """W: work-groups per KV head, at most B * S (the launch caps it at one round of the
    device's resident work-groups)."""
    B = len(lens)
    W = B * S if W is None else W
    assert 1 <= W <= B * S
    T, budget, first = plan(lens, Nk, window, W)
    total = T[B]
    written = {}
    keys = {b: [] for b in range(B)}
    for w in range(W):
        g_lo = w * budget
        if g_lo >= total:
            assert w not in first
            continue
        g_hi = min(total, g_lo + budget)
        b = first[w]
        assert T[b] <= g_lo < T[b + 1]
        while True:
            vis, n = visible(lens[b], Nk, window)
            t_lo = max(0, max(T[b], g_lo) - T[b] - PIECE)
            t_hi = max(0, min(T[b + 1], g_hi) - T[b] - PIECE)
            start, hi = vis + t_lo * TILE, min(n, vis + t_hi * TILE)
            # a piece is empty only when the run ends inside the virtual tiles
            assert (t_hi > t_lo and start < hi) or (t_hi == t_lo == 0 and min(T[b + 1], g_hi) - T[b] <= PIECE)
            keys[b].extend(range(start, hi))
            idx = w + b
            assert idx not in written and idx < B * (S + 1)
            written[idx] = b
            if T[b + 1] >= g_hi:
                break
            b += 1
            while T[b + 1] == T[b]:  # skip sequences with no visible key
                b += 1
    for b in range(B):
        vis, n = visible(lens[b], Nk, window)
        assert keys[b] == list(range(vis, n)), b
        if T[b + 1] > T[b]:
            w_lo, w_hi = T[b] // budget, (T[b + 1] - 1) // budget
            reads = [w + b for w in range(w_lo, w_hi + 1)]
        else:
            reads = []
        assert reads == sorted(i for i, bb in written.items() if bb == b), b
    return len(written)


@pytest.mark.parametrize("seed", range(8))
def test_plan_covers_keys_once_with_unique_partials(seed):
    rng = random.Random(seed)
    for _ in range(150):
        B = rng.choice([1, 2, 3, 5, 16, 64, 300])
        Nk = rng.choice([1, 7, 128, 129, 1000, 4096, 32768])
        S = rng.choice([1, 2, 3, 7, 16, 64])
        if S > Nk:
            continue
        window = rng.choice([0, 0, 1, 40, 200, 4096])
        lens = [rng.choice([0, 1, Nk, rng.randint(0, Nk)]) for _ in range(B)]
        run_plan(lens, Nk, window, S)
        run_plan(lens, Nk, window, S, W=rng.randint(1, B * S))


def test_plan_equal_full_lengths():
    """Equal lengths: every work-group's run is budget units, so a sequence of 32
    tiles and its virtual one (33 units) are spread over the 24 work-groups of three
    sequences in runs of 5 units; the two runs that cross a boundary write two
    partials each."""
    B, Nk, S = 3, 4096, 8
    T, budget, first = plan([Nk] * B, Nk, 0, B * S)
    assert T == [0, 33, 66, 99] and budget == 5
    assert sorted(first.items()) == [(w, (5 * w) // 33) for w in range(20)]
    assert run_plan([Nk] * B, Nk, 0, S) == 20 + 2


def test_plan_long_sequence_among_short_ones():
    """One long sequence among one-key ones is spread over many work-groups."""
    lens = [20000] + [1] * 31
    T, budget, _ = plan(lens, 20000, 0, 32 * 16)
    assert budget == 1
    # one work-group per unit: 157 tiles and a virtual one for the long sequence,
    # a virtual and a real one for each one-key sequence
    assert T[-1] == 158 + 31 * 2
    assert run_plan(lens, 20000, 0, 16) == 158 + 31 * 2
