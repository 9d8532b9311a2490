"""The forward's two chains of query tiles (bsm_fwd_step_chain): the ring run as
two chains on two streams gives the one-launch ring's state, O and LSE bit for
bit; the chains cover every tile with work once, a sample's tiles in one chain."""
import numpy as np
import pytest
import torch

import block_sparse_masked_metadata_amd as bsm
from workloads import config, random_small, packed_text, packed_multimodal
from gpu_common import Case, needs_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not needs_gpu, reason="needs a GPU")]


def _random(seed, ranks=4, order="ptrr"):
    rng = np.random.default_rng(seed)
    lay = random_small(rng, 128 * ranks * 4, max_span=300)
    lay.ranks, lay.order, lay.seed = ranks, order, seed
    lay.hq, lay.hkv, lay.d = 4, 2, 128
    return lay


def _both(case):
    one = case.ring(chains=1)
    two = case.ring(chains=2)
    st1 = case.ring(chains=1, keep_state=True)[2]
    st2 = case.ring(chains=2, keep_state=True)[2]
    torch.cuda.synchronize()
    return one, two, st1, st2


@pytest.mark.parametrize("maker", ["packed_text", "packed_multimodal", "video_group", "sliding_window", "long_mixed",
                                   "random5", "random6"])
def test_two_chains_equal_one_launch(maker):
    """Every workload's full share, including the two whose rule picks one
    chain (sliding window 128K, long mixed 1M): the split by samples is
    exercised on them too."""
    lay = {"packed_text": packed_text, "packed_multimodal": packed_multimodal,
           "video_group": lambda: config(6), "sliding_window": lambda: config(4),
           "long_mixed": lambda: config(5)}.get(maker)
    lay = lay() if lay else _random(int(maker[-1]))
    case = Case(lay)
    one, two, st1, st2 = _both(case)
    assert torch.equal(one[0], two[0]) and torch.equal(one[1], two[1])
    for a, b in zip(st1, st2):
        assert torch.equal(a, b)


def test_two_chains_dense_call_plan():
    case = Case(_random(7), dense=True)
    one, two, _, _ = _both(case)
    assert torch.equal(one[0], two[0]) and torch.equal(one[1], two[1])


def test_chains_cover_tiles_once_by_sample():
    """Chain 0 alone writes exactly its tiles' rows; chain 1 then the rest.
    The tiles of one sample (by a tile's first row) share a chain."""
    lay = packed_multimodal()
    case = Case(lay)
    info = case.dp.info
    R, S, T = case.R, case.S, (case.S + 127) // 128
    steps = [s for s in range(R) if info["fwd_items"][s] > 0]
    assert all(0 <= info["fwd_chain0_items"][s] <= info["fwd_items"][s] for s in range(R))
    assert any(0 < info["fwd_chain0_items"][s] < info["fwd_items"][s] for s in steps)
    o = torch.full((S, case.hq, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((case.hq, S), float("nan"), dtype=torch.float32, device="cuda")
    st = bsm.new_state(S, case.hq, 128)
    for chain in (0, 1):
        for s in steps:
            j = (case.r - s) % R
            bsm.fwd_step(case.dp, s, case.heads, case.q, case.k_shards[j], case.v_shards[j], st, o, lse,
                         chain=chain)
        torch.cuda.synchronize()
        written = torch.isfinite(lse).any(dim=0).cpu().numpy()
        tiles = np.array([written[a * 128:(a + 1) * 128].any() for a in range(T)])
        if chain == 0:
            chain0 = tiles.copy()
            assert chain0.any() and not chain0.all()
        else:
            assert tiles.all()
    ref_o, ref_lse, _ = case.ring(chains=1)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse)
    sample = lay.tracks()[0][case.rows]
    first = {}
    for a in range(T):
        g = int(sample[a * 128])
        assert first.setdefault(g, chain0[a]) == chain0[a], f"sample {g} split over both chains"


def test_chain_argument_checked():
    case = Case(packed_text())
    st = bsm.new_state(case.S, case.hq, 128)
    o = torch.empty(case.S, case.hq, 128, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(case.hq, case.S, dtype=torch.float32, device="cuda")
    with pytest.raises(bsm.BsmError) as e:
        bsm.fwd_step(case.dp, 0, case.heads, case.q, case.k_shards[case.r], case.v_shards[case.r], st, o, lse,
                     chain=2)
    assert e.value.code == bsm._capi.BSM_E_INVALID and "chain" in str(e.value)


def test_fwd_chains_rule():
    """Two chains exactly when every step with work gives each chain between
    one and CHAIN_MAX_ROUNDS rounds of workgroups (two per CU)."""
    from block_sparse_masked_metadata_amd.ring import CHAIN_MAX_ROUNDS
    full = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    for lay in (packed_text(), packed_multimodal(), _random(5)):
        case = Case(lay)
        info = case.dp.info
        ok = []
        for s in range(case.R):
            n, c0 = info["fwd_items"][s], info["fwd_chain0_items"][s]
            if n:
                ok.append(min(c0, n - c0) * case.hq >= full and max(c0, n - c0) * case.hq <= CHAIN_MAX_ROUNDS * full)
        assert bsm.fwd_chains(case.dp, case.heads) == (2 if ok and all(ok) else 1)
