"""Dense calls (MARBLE section 03, "Chunked ring attention": each ring step as
a few full / causal / reverse-causal calls that compute every legal pair
exactly once): the planner's calls against the oracle's mask, by brute force."""
import dataclasses

import numpy as np
import pytest

import block_sparse_masked_metadata_amd as bsm
from workloads import config, random_small
from oracle.mask import legal, take

FULL, CAUSAL, REVERSE, PAST = 0, 1, 2, 3


def _relation(kind, pq, pk, w):
    """The header's relations, written out over position grids."""
    d = pq[:, None] - pk[None, :]
    if kind == FULL:
        return np.ones(d.shape, bool)
    if kind == CAUSAL:
        return (d >= 0) & (d < w)
    if kind == REVERSE:
        return d < 0
    assert kind == PAST
    return d >= w


def _check_cover(lay, plan, r, s):
    R, S = plan.info["ranks"], plan.info["shard_tokens"]
    perm = plan.permutation().astype(np.int64)
    j = (r - s) % R
    qtok, ktok = perm[r * S:(r + 1) * S], perm[j * S:(j + 1) * S]
    tr = lay.tracks()
    want = legal(take(tr, qtok), take(tr, ktok), lay.window)
    pos = np.asarray(tr[3], np.int64)
    cnt = np.zeros(want.shape, np.int32)
    calls = plan.dense_calls(r, s)
    for q0, qn, k0, kn, kind in calls:
        assert qn >= 1 and kn >= 1 and q0 >= 0 and k0 >= 0 and q0 + qn <= S and k0 + kn <= S
        cnt[q0:q0 + qn, k0:k0 + kn] += _relation(kind, pos[qtok[q0:q0 + qn]], pos[ktok[k0:k0 + kn]],
                                                 lay.window)
    assert cnt.max(initial=0) <= 1, "a pair is computed twice"
    assert np.array_equal(cnt.astype(bool), want), "calls differ from the mask"
    return calls


@pytest.mark.parametrize("seed", range(16))
def test_calls_cover_mask_exactly_random(seed):
    rng = np.random.default_rng(1500 + seed)
    R = int(rng.integers(1, 5))
    lay = random_small(rng, 16 * R * int(rng.integers(1, 6)), max_span=int(rng.choice([6, 20, 60])))
    for order in ("contiguous", "ptrr"):
        plan = bsm.Plan(lay.tracks(), lay.window, R, block=16, order=order)
        for r in range(R):
            for s in range(R):
                _check_cover(lay, plan, r, s)


def test_calls_cover_mask_chunked_order():
    rng = np.random.default_rng(77)
    R = 3
    lay = random_small(rng, 16 * R * 8, max_span=40)
    base = bsm.Plan(lay.tracks(), lay.window, R, block=16, order="contiguous")
    perm, _ = base.chunk_order(2, 4, 0.0, 2)
    plan = bsm.Plan(lay.tracks(), lay.window, R, block=16, order="explicit", explicit_block_perm=perm)
    for r in range(R):
        for s in range(R):
            _check_cover(lay, plan, r, s)


@pytest.mark.parametrize("c", [1, 2, 3])
def test_calls_cover_mask_workloads(c):
    lay = config(c)
    plan = bsm.Plan.from_layout(lay)
    r = plan.info["busiest_rank"]
    for s in sorted({0, 1, lay.ranks - 1}):
        calls = _check_cover(lay, plan, r, s)
        _, pairs = plan.step_map(r, s)
        assert (len(calls) > 0) == (pairs > 0)


def test_bidirectional_span_is_causal_plus_reverse():
    # one sample, one bidirectional span, one rank: exactly one causal and one
    # reverse call over the whole span (the diagonal split of a full block)
    n = 64
    tr = (np.zeros(n, np.int32), np.zeros(n, np.int32), -np.ones(n, np.int32), np.arange(n, dtype=np.int32))
    plan = bsm.Plan(tr, 0x7FFFFFFF, 1, block=16, order="contiguous")
    calls = plan.dense_calls(0, 0)
    assert sorted(map(tuple, calls.tolist())) == [(0, n, 0, n, CAUSAL), (0, n, 0, n, REVERSE)]


def test_noise_span_of_one_seg_is_full():
    # text, then a noise span of its own seg: the span's queries see the text
    # causally and the whole span fully; no reverse call is needed for it
    n = 48
    smp = np.zeros(n, np.int32)
    seg = np.array([-1] * 16 + [3] * 32, np.int32)
    noise = np.array([-1] * 16 + [0] * 32, np.int32)
    tr = (smp, seg, noise, np.arange(n, dtype=np.int32))
    plan = bsm.Plan(tr, 0x7FFFFFFF, 1, block=16, order="contiguous")
    calls = sorted(map(tuple, plan.dense_calls(0, 0).tolist()))
    assert (16, 32, 16, 32, FULL) in calls
    assert all(c[4] != REVERSE for c in calls)
    lay = dataclasses.make_dataclass("L", ["window"])(0x7FFFFFFF)
    lay.tracks = lambda: tr
    _check_cover(lay, plan, 0, 0)


def test_dense_device_plan_packs_on_host():
    lay = config(3)
    plan = bsm.Plan.from_layout(lay)
    r = plan.info["busiest_rank"]
    assert bsm._capi.bsm_dplan_calls_bytes(plan.handle, r) > 0
    with pytest.raises(bsm.BsmError):
        bsm._capi.bsm_plan_dense_calls(plan.handle, r, lay.ranks)


def test_dense_device_plan_refuses_huge_positions():
    n = 32
    tr = (np.zeros(n, np.int32), -np.ones(n, np.int32), -np.ones(n, np.int32),
          np.arange(0x7FFFFFFF - n + 1, 0x7FFFFFFF + 1, dtype=np.int64).astype(np.int32))
    plan = bsm.Plan(tr, 0x7FFFFFFF, 1, block=16, order="contiguous")
    with pytest.raises(bsm.BsmError) as e:
        bsm._capi.bsm_dplan_calls_bytes(plan.handle, 0)
    assert e.value.code == bsm._capi.BSM_E_UNSUPPORTED
