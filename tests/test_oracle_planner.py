"""Pins of the oracle planner (oracle/planner.py)."""
import numpy as np
import pytest

from workloads import random_small, packed_text, sliding_window, long_mixed, WINDOW_INF
from oracle import planner
from oracle.planner import EMPTY, PARTIAL, FULL
from goldens import read


def _pylegal(tr, w, q, k):
    s, g, nz, p = (a.tolist() for a in tr)
    d = p[q] - p[k]
    return ((0 <= d < w) or (g[q] == g[k] and g[k] >= 0)) and \
        (nz[k] < 0 or nz[q] == nz[k]) and s[q] == s[k]


@pytest.mark.parametrize("seed", range(12))
def test_maps_match_pure_python_enumeration(seed):
    rng = np.random.default_rng(1000 + seed)
    ranks = [1, 2, 3, 4][seed % 4]
    block = [4, 8, 16][seed % 3]
    order = ["contiguous", "ptrr"][seed % 2]
    n = block * ranks * int(rng.integers(1, 4))
    if order == "contiguous" and seed % 3 == 0:
        n += ranks  # ragged last tile in each shard
    lay = random_small(rng, n)
    tr = lay.tracks()
    p = planner.build(tr, lay.window, ranks, block, order)
    s_tok = n // ranks
    for r in range(ranks):
        for s in range(ranks):
            j = (r - s) % ranks
            mp, tot = p.step_map(r, s)
            want_tot = 0
            for a in range(p.tiles_per_shard):
                qa = p.perm[r * s_tok + a * block: min(r * s_tok + (a + 1) * block, (r + 1) * s_tok)]
                for b in range(p.tiles_per_shard):
                    kb = p.perm[j * s_tok + b * block: min(j * s_tok + (b + 1) * block, (j + 1) * s_tok)]
                    c = sum(_pylegal(tr, lay.window, int(x), int(y)) for x in qa for y in kb)
                    want = EMPTY if c == 0 else (FULL if c == len(qa) * len(kb) else PARTIAL)
                    assert mp[a, b] == want
                    want_tot += c
            assert tot == want_tot


def _causal_single(n):
    return (np.zeros(n, np.int32), -np.ones(n, np.int32), -np.ones(n, np.int32),
            np.arange(n, dtype=np.int32))


def test_causal_contiguous_block_counts():
    """Ring-attention explainer: causal with 4 contiguous devices -> 1,2,3,4 blocks."""
    g = read("ring_explainer_block_counts.txt")
    want = [int(x) for x in g["contiguous"].split()]
    n = 64
    p = planner.build(_causal_single(n), WINDOW_INF, 4, n // 4, "contiguous")
    got = [sum(int(p.step_map(r, s)[0].astype(bool).sum()) for s in range(4)) for r in range(4)]
    assert got == want
    # the diagonal block is the only partial one
    for r in range(4):
        assert p.step_map(r, 0)[0][0, 0] == PARTIAL
        for s in range(1, r + 1):
            assert p.step_map(r, s)[0][0, 0] == FULL


def test_zigzag_block_counts():
    """Ring-attention explainer: zigzag chunks (p, 2P-1-p) -> 9 chunk-pairs each."""
    g = read("ring_explainer_block_counts.txt")
    chunks = [tuple(int(c) for c in x.split(",")) for x in g["zigzag_chunks"].split()]
    want = [int(x) for x in g["zigzag"].split()]
    n = 64
    perm = [c for pair in chunks for c in pair]
    p = planner.build(_causal_single(n), WINDOW_INF, 4, n // 8, "explicit", perm)
    got = [sum(int(p.step_map(r, s)[0].astype(bool).sum()) for s in range(4)) for r in range(4)]
    assert got == want


def test_packed_text_pairs_closed_form():
    """Block-diagonal causal: total legal pairs = sum over documents l(l+1)/2."""
    lay = packed_text(n=8192, seed=2, ranks=8)
    p = planner.build(lay.tracks(), lay.window, 8, 128, "ptrr")
    lens = np.array([b - a for a, b, _, _ in lay.spans], np.int64)
    assert int(p.cost.sum()) == int((lens * (lens + 1) // 2).sum())
    assert int(p.rank_pairs().sum()) == int(p.cost.sum())


def test_long_mixed_pairs_closed_form():
    """Text l(l+1)/2 per document plus l^2 per bidirectional clip."""
    lay = long_mixed(n=65536, seed=5, ranks=8, clip=4096)
    p = planner.build(lay.tracks(), lay.window, 8, 128, "ptrr")
    want = 0
    for a, b, mode, _ in lay.spans:
        ln = b - a
        want += ln * ln if mode == "full" else ln * (ln + 1) // 2
    assert int(p.cost.sum()) == want


def test_sliding_window_map_closed_form():
    """Clips of C tokens, window W, contiguous shards = clips, 128-token tiles.
    Step 0: every tile full.  Step 1 (previous clip, same document): q tile a
    (a < W/128) is full for b > a + C/128 - W/128, partial at b = a + C/128 - W/128,
    empty otherwise; q tiles a >= W/128 empty.  Later steps empty.  Pair counts:
    C^2 + (W-1)W/2 for a rank with a predecessor in its document."""
    clip, w, tb = 2048, 512, 128
    lay = sliding_window(n=8 * clip, clip=clip, clips_per_doc=4, window=w, ranks=8)
    p = planner.build(lay.tracks(), lay.window, 8, tb, "contiguous")
    tiles = clip // tb
    wt = w // tb
    pairs = p.rank_pairs()
    for r in range(8):
        m0, _ = p.step_map(r, 0)
        assert np.all(m0 == FULL)
        m1, _ = p.step_map(r, 1)
        if r % 4 == 0:
            assert np.all(m1 == EMPTY)
            assert pairs[r].sum() == clip * clip
        else:
            want = np.zeros((tiles, tiles), np.uint8)
            for a in range(wt):
                want[a, a + tiles - wt] = PARTIAL
                want[a, a + tiles - wt + 1:] = FULL
            assert np.array_equal(m1, want)
            assert pairs[r].sum() == clip * clip + (w - 1) * w // 2
        for s in range(2, 8):
            assert not p.step_map(r, s)[0].any()
    assert p.busiest_rank() == 1


def test_ptrr_invariants():
    lay = packed_text(n=16384, seed=4, ranks=8)
    p = planner.build(lay.tracks(), lay.window, 8, 128, "ptrr")
    t = len(p.starts)
    assert sorted(p.tiles_new.tolist()) == list(range(t))
    per = t // 8
    for r in range(8):
        mine = p.tiles_new[r * per:(r + 1) * per]
        assert np.all(np.diff(mine) > 0)          # sequence order within a rank
    # perm is a bijection of tokens
    assert np.array_equal(np.sort(p.perm), np.arange(lay.n))
    # balance: the busiest rank is close to the mean (MARBLE reports within 0.1%
    # on its masks); contiguous shards are far worse on the same layout
    tot = np.array([p.cost[p.tiles_new[r * per:(r + 1) * per]].sum() for r in range(8)])
    pc = planner.build(lay.tracks(), lay.window, 8, 128, "contiguous")
    totc = np.array([pc.cost[r * per:(r + 1) * per].sum() for r in range(8)])
    assert tot.max() / tot.mean() < totc.max() / totc.mean()
    assert tot.max() / tot.mean() < 1.05


def test_ptrr_deal_snake():
    """Rounds of R, every other round reversed: with strictly decreasing costs
    block i goes to rank i in even rounds and R-1-i in odd rounds."""
    cost = np.arange(16)[::-1] * 10
    owner = planner.ptrr_owner(cost, 4)
    assert owner.tolist() == [0, 1, 2, 3, 3, 2, 1, 0, 0, 1, 2, 3, 3, 2, 1, 0]
    # ties keep the lower index first
    owner = planner.ptrr_owner(np.zeros(8, np.int64), 4)
    assert owner.tolist() == [0, 1, 2, 3, 3, 2, 1, 0]
