"""Sparse fetch (MARBLE section 04, "Sparse all-to-all and strategy selection"):
the remote key tiles a rank needs, against the planner's own tile maps and
against closed forms of the layouts."""
import numpy as np
import pytest

import block_sparse_masked_metadata_amd as bsm
from workloads import config, random_small


def _from_maps(plan, r):
    R = plan.info["ranks"]
    T = plan.info["tiles_per_shard"]
    need = np.zeros((R, T), np.uint8)
    for s in range(1, R):
        mp, _ = plan.step_map(r, s)
        need[(r - s) % R] |= (mp > 0).any(axis=0).astype(np.uint8)
    return need


@pytest.mark.parametrize("seed", range(12))
def test_fetch_set_equals_union_of_step_maps_random(seed):
    rng = np.random.default_rng(300 + seed)
    R = int(rng.integers(2, 6))
    lay = random_small(rng, 16 * R * int(rng.integers(2, 6)))
    for order in ("contiguous", "ptrr"):
        plan = bsm.Plan(lay.tracks(), lay.window, R, block=16, order=order)
        for r in range(R):
            need, cnt = plan.fetch_set(r)
            want = _from_maps(plan, r)
            assert np.array_equal(need, want)
            assert cnt == int(want.sum())
            assert not need[r].any()


@pytest.mark.parametrize("c", [2, 3])
def test_fetch_set_workloads(c):
    lay = config(c)
    for order in (lay.order, "contiguous"):
        plan = bsm.Plan(lay.tracks(), lay.window, lay.ranks, 128, order)
        r = plan.info["busiest_rank"]
        need, cnt = plan.fetch_set(r)
        assert np.array_equal(need, _from_maps(plan, r))


def test_sliding_window_closed_form():
    # 8 clips of 16384 tokens, 4 clips per document, window 4096 = 32 tiles:
    # a clip that is not its document's first needs the previous clip's last
    # 32 tiles and nothing else; a document's first clip needs nothing
    lay = config(4)
    plan = bsm.Plan.from_layout(lay)
    T = plan.info["tiles_per_shard"]
    for r in range(lay.ranks):
        need, cnt = plan.fetch_set(r)
        want = np.zeros_like(need)
        if r % 4:
            want[r - 1, T - 32:] = 1
        assert np.array_equal(need, want), r
        assert cnt == (32 if r % 4 else 0)


def test_fetch_rows_layout():
    lay = config(4)
    plan = bsm.Plan.from_layout(lay)
    S = plan.info["shard_tokens"]
    src = bsm.fetch_rows(plan, 1)
    assert len(src) == S + 32 * 128
    assert np.array_equal(src[:S], np.arange(S, 2 * S))
    assert np.array_equal(src[S:], np.arange(S - 32 * 128, S))
