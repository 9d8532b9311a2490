"""Key intervals of the host planner (MARBLE section 03, "Block classification":
a partial tile may test one range per key) against the oracle predicate.

For every key with a range, the queries it is legal for must be exactly the
tokens whose index (in the order the plan was given) lies in [lo, hi); a key
without one must really have a legal set that is not one run of tokens.
Brute force over random all-mode layouts, the same layouts in vision-group
order (positions then no longer rise with the index), and sampled keys of the
workloads."""
import numpy as np
import pytest

import block_sparse_masked_metadata_amd as bsm
from oracle.mask import legal, take
from workloads import config, random_small


def _runs(mask):
    """Number of maximal runs of True."""
    m = np.concatenate([[False], mask, [False]])
    return int((np.diff(m.astype(np.int8)) == 1).sum())


def _check_keys(lay, keys, lo, hi):
    tr = lay.tracks()
    sample = np.asarray(tr[0])
    for k in keys:
        # the legal set lies inside the key's sample: test that sample's queries
        qs = np.flatnonzero(sample == sample[k])
        got = legal(take(tr, qs), take(tr, [k]), lay.window)[:, 0]
        if hi[k] >= lo[k]:
            want = (qs >= lo[k]) & (qs < hi[k])
            assert np.array_equal(got, want), (lay.name, int(k), int(lo[k]), int(hi[k]))
        else:
            assert _runs(got) > 1, (lay.name, int(k))


@pytest.mark.parametrize("seed", range(40))
def test_intervals_random_layouts(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(8, 160))
    lay = random_small(rng, n)
    plan = bsm.Plan(lay.tracks(), lay.window, 1, block=16, order="contiguous")
    lo, hi = plan.key_intervals()
    assert plan.info["interval_keys"] == int((hi >= lo).sum())
    _check_keys(lay, range(n), lo, hi)


@pytest.mark.parametrize("seed", range(30))
def test_intervals_random_layouts_vision_group_order(seed):
    """The same brute force after the vision-group order: positions no longer
    rise with the index, and the coordinate of the ranges is the new index."""
    from workloads import permuted
    rng = np.random.default_rng(1100 + seed)
    n = int(rng.integers(8, 200))
    base = random_small(rng, n, max_span=20)
    lay = permuted(base, bsm.vision_group_order(base.tracks()))
    plan = bsm.Plan(lay.tracks(), lay.window, 1, block=16, order="contiguous")
    lo, hi = plan.key_intervals()
    assert plan.info["interval_keys"] == int((hi >= lo).sum())
    _check_keys(lay, range(n), lo, hi)


@pytest.mark.parametrize("c", [1, 2, 3, 4])
def test_intervals_workloads_sampled(c):
    lay = config(c)
    plan = bsm.Plan.from_layout(lay)
    lo, hi = plan.key_intervals()
    rng = np.random.default_rng(c)
    keys = rng.choice(lay.n, size=min(lay.n, 300), replace=False)
    # also every key that has no range
    keys = np.unique(np.concatenate([keys, np.flatnonzero(hi < lo)[:300]]))
    _check_keys(lay, keys, lo, hi)


def test_interval_counts_of_workloads():
    # Closed forms of the layouts: text, clips and generated images have one
    # range per key; the second image of a bidirectional pair is seen by the
    # first image and by every later token, with text in between (two runs).
    lay = config(3)
    plan = bsm.Plan.from_layout(lay)
    lo, hi = plan.key_intervals()
    seg = np.asarray(lay.tracks()[1])
    noise = np.asarray(lay.tracks()[2])
    # keys of the later span of a group that are not generated images
    later = np.zeros(lay.n, bool)
    for g in np.unique(seg[seg >= 0]):
        idx = np.flatnonzero(seg == g)
        runs = np.split(idx, np.flatnonzero(np.diff(idx) > 1) + 1)
        for r in runs[1:]:
            later[r] = True
    expect_none = later & (noise < 0)
    assert np.array_equal(hi < lo, expect_none)
    for c in (2, 4):
        p = bsm.Plan.from_layout(config(c))
        assert p.info["interval_keys"] == config(c).n
