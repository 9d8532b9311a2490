"""Chunked ring layouts (MARBLE section 03, "Chunked ring attention"): the
planner's chunk search against an independent evaluation of its cost and of
the layouts it can produce."""
import itertools

import numpy as np
import pytest

import block_sparse_masked_metadata_amd as bsm
from workloads import config, random_small


def _cost(plan):
    """sum over steps of the slowest rank, from the rebuilt plan's pair matrix"""
    P = plan.pairs()
    R = P.shape[0]
    return sum(max(int(P[r][s]) for r in range(R)) for s in range(R))


def _chunks_of(perm, R, k):
    """Each rank's blocks must be k whole chunks of the original order."""
    nt = len(perm)
    ct = nt // (R * k)
    per = nt // R
    owners = []
    for r in range(R):
        blocks = np.sort(perm[r * per:(r + 1) * per])
        assert np.array_equal(perm[r * per:(r + 1) * per], blocks)  # ascending within a rank
        chunks = set(blocks // ct)
        assert len(chunks) == k and all(set(blocks[blocks // ct == c]) == set(range(c * ct, (c + 1) * ct))
                                        for c in chunks)
        owners.append(sorted(chunks))
    return owners


@pytest.mark.parametrize("seed", range(8))
def test_chunk_search_cost_matches_rebuilt_plan(seed):
    rng = np.random.default_rng(700 + seed)
    R = int(rng.integers(2, 5))
    tps = 8
    lay = random_small(rng, 16 * R * tps)
    base = bsm.Plan(lay.tracks(), lay.window, R, block=16, order="contiguous")
    for tau in (0.0, 50.0):
        perm, info = base.chunk_order(1, 8, tau, 2)
        assert sorted(perm.tolist()) == list(range(R * tps))
        _chunks_of(perm, R, info["chunks_per_rank"])
        ch = bsm.Plan(lay.tracks(), lay.window, R, block=16, order="explicit", explicit_block_perm=perm)
        assert info["step_max_sum"] == _cost(ch)
        assert info["range_term"] == pytest.approx(tau * R * info["chunks_per_rank"])
        assert info["cost"] == pytest.approx(info["step_max_sum"] + info["range_term"])


def test_one_chunk_in_sequence_order_is_contiguous():
    lay = config(3)
    base = bsm.Plan(lay.tracks(), lay.window, lay.ranks, 128, "contiguous")
    perm, info = base.chunk_order(1, 1, 0.0, 0)
    # strategy 1 deals chunk r to rank r; strategy 0 sorts by work: the cheaper wins
    ch = bsm.Plan(lay.tracks(), lay.window, lay.ranks, 128, "explicit", explicit_block_perm=perm)
    assert info["step_max_sum"] == _cost(ch)
    assert info["step_max_sum"] <= _cost(base)


def test_chunk_search_is_minimal_over_tiny_assignments():
    # R = 2, k = 1 or 2 over 4 chunks: the best dealt candidate is never worse
    # than the best of all balanced assignments by more than the swap search allows;
    # with swaps the search reaches the optimum here.
    rng = np.random.default_rng(5)
    lay = random_small(rng, 16 * 2 * 4)
    base = bsm.Plan(lay.tracks(), lay.window, 2, block=16, order="contiguous")
    perm, info = base.chunk_order(2, 2, 0.0, 8)
    best = None
    for a in itertools.combinations(range(4), 2):
        own = [0 if c in a else 1 for c in range(4)]
        order = [c for r in range(2) for c in range(4) if own[c] == r]
        p = np.concatenate([np.arange(2 * c, 2 * c + 2) for c in order]).astype(np.int32)
        pl = bsm.Plan(lay.tracks(), lay.window, 2, block=16, order="explicit", explicit_block_perm=p)
        c = _cost(pl)
        best = c if best is None else min(best, c)
    assert info["step_max_sum"] == best


def test_tau_prefers_fewer_ranges():
    lay = config(2)
    base = bsm.Plan(lay.tracks(), lay.window, lay.ranks, 128, "contiguous")
    _, free = base.chunk_order(1, 32, 0.0, 0)
    _, dear = base.chunk_order(1, 32, 1e12, 0)
    assert dear["chunks_per_rank"] == 1
    assert free["step_max_sum"] <= dear["step_max_sum"]


def test_chunk_search_errors():
    lay = config(2)
    base = bsm.Plan(lay.tracks(), lay.window, lay.ranks, 128, "contiguous")
    for args in ((0, 4, 0.0, 0), (4, 2, 0.0, 0), (1, 4, -1.0, 0), (1, 4, 0.0, -1)):
        with pytest.raises(bsm.BsmError):
            base.chunk_order(*args)
