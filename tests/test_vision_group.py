"""The vision-group layout transform (MARBLE section 04, "Layout transforms":
text first, then the group spans in reverse, so that each key's visible
queries form one range; the page reports partial tiles falling from 49% to
4% on Molmo2 video).  CPU checks: the order's structure, the one-range claim
by brute force with the oracle's mask, the planner against the oracle planner
on transformed layouts (positions no longer rise with the index), and the
partial-tile fraction before and after on a synthetic video layout."""
import numpy as np
import pytest

import block_sparse_masked_metadata_amd as bsm
from block_sparse_masked_metadata_amd import _capi as C
from oracle.mask import legal, take
from workloads import random_small, video_group, permuted
from test_capi_host import _compare


def _runs(mask):
    m = np.concatenate([[False], mask, [False]])
    return int((np.diff(m.astype(np.int8)) == 1).sum())


@pytest.mark.parametrize("seed", range(12))
def test_order_structure(seed):
    """A bijection that keeps every sample in place; per sample the tokens of
    spans whose seg id has two or more runs come last, in reverse span order,
    and every other token keeps its relative order."""
    rng = np.random.default_rng(2000 + seed)
    lay = random_small(rng, int(rng.integers(20, 400)), max_span=30)
    perm = bsm.vision_group_order(lay.tracks()).astype(np.int64)
    n = lay.n
    assert np.array_equal(np.sort(perm), np.arange(n))
    assert np.array_equal(lay.sample[perm], lay.sample)          # samples stay where they were
    for sid in np.unique(lay.sample):
        idx = np.flatnonzero(lay.sample == sid)
        seg = lay.seg[idx]
        starts = np.flatnonzero(np.concatenate([[True], seg[1:] != seg[:-1]]))
        runs = [(idx[a], idx[b - 1] + 1) for a, b in zip(starts, list(starts[1:]) + [len(idx)])]
        ids, counts = np.unique([lay.seg[a] for a, _ in runs if lay.seg[a] >= 0], return_counts=True)
        group_ids = set(ids[counts >= 2].tolist())
        grp = [r for r in runs if lay.seg[r[0]] in group_ids]
        rest = np.array([t for t in idx if lay.seg[t] not in group_ids], np.int64)
        want = np.concatenate([rest] + [np.arange(a, b) for a, b in reversed(grp)]).astype(np.int64)
        assert np.array_equal(perm[idx], want)


@pytest.mark.parametrize("seed", range(6))
def test_every_key_one_range_on_video(seed):
    """The page's claim, by brute force with the oracle's mask: on video
    samples (causal text, one bidirectional group of frames per sample) every
    key's visible queries are one run of the transformed order, while in the
    original order most frame keys see several runs."""
    lay = video_group(n=6000, seed=seed, frame=24, stamp=3, min_frames=2, max_frames=9)
    lay_v = permuted(lay, bsm.vision_group_order(lay.tracks()))
    for L, expect_one in ((lay, False), (lay_v, True)):
        tr = L.tracks()
        multi = 0
        for sid in np.unique(L.sample):
            qs = np.flatnonzero(L.sample == sid)
            m = legal(take(tr, qs), take(tr, qs), L.window)       # [queries, keys]
            multi += sum(_runs(m[:, j]) > 1 for j in range(len(qs)))
        if expect_one:
            assert multi == 0
        else:
            assert multi > 0.5 * int((L.seg >= 0).sum())


@pytest.mark.parametrize("seed", range(10))
def test_planner_matches_oracle_on_transformed_random(seed):
    rng = np.random.default_rng(2100 + seed)
    ranks = [1, 2, 3, 4][seed % 4]
    block = [8, 16][seed % 2]
    order = ["contiguous", "ptrr"][(seed // 2) % 2]
    n = block * ranks * int(rng.integers(2, 6))
    base = random_small(rng, n, max_span=25)
    lay = permuted(base, bsm.vision_group_order(base.tracks()))
    _compare(lay, ranks, block, order)


def test_planner_matches_oracle_on_transformed_video():
    lay = video_group(n=16384, frame=64, stamp=4, min_frames=4, max_frames=20)
    lay_v = permuted(lay, bsm.vision_group_order(lay.tracks()))
    _compare(lay_v, 8, 128, "ptrr")


def test_partial_tiles_fall_on_video():
    """Synthetic video at 128K tokens: 45.5% of the non-empty tile pairs are
    partial in the original order, 5.3% in vision-group order (the page: 49%
    and 4% on Molmo2 video at 512K), every key gets a range, and the legal
    pairs are the same."""
    lay = video_group()
    before = bsm.Plan.from_layout(lay).info
    after = bsm.Plan.from_layout(permuted(lay, bsm.vision_group_order(lay.tracks()))).info
    frac = lambda i: i["partial_tiles"] / (i["partial_tiles"] + i["full_tiles"])
    print(f"partial tiles: {frac(before):.3f} -> {frac(after):.3f}; keys with a range "
          f"{before['interval_keys']} -> {after['interval_keys']} of {lay.n}")
    assert after["total_pairs"] == before["total_pairs"]
    assert frac(before) > 0.4 and frac(after) < 0.06
    assert after["interval_keys"] == lay.n


def test_dense_calls_need_rising_positions():
    lay = video_group(n=8192, frame=64, stamp=4, min_frames=4, max_frames=8)
    plan = bsm.Plan.from_layout(permuted(lay, bsm.vision_group_order(lay.tracks())))
    with pytest.raises(bsm.BsmError) as e:
        plan.dense_calls(0, 0)
    assert e.value.code == C.BSM_E_UNSUPPORTED
    with pytest.raises(bsm.BsmError) as e:
        C.bsm_dplan_calls_bytes(plan.handle, 0)
    assert e.value.code == C.BSM_E_UNSUPPORTED


def test_invalid_tracks_are_refused():
    n = 16
    s = np.zeros(n, np.int32)
    s[3] = 1
    with pytest.raises(bsm.BsmError) as e:
        C.bsm_vision_group_order(s, -np.ones(n, np.int32))
    assert e.value.code == C.BSM_E_INVALID
    with pytest.raises(bsm.BsmError):
        C.bsm_vision_group_order(np.full(n, -1, np.int32), -np.ones(n, np.int32))
