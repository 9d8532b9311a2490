"""Sparse fetch on the GPU (MARBLE section 04, "Sparse all-to-all and strategy
selection"): one pass over the rank's shard and its fetched remote tiles is
bitwise the single pass over all shards (same tiles, same order), on PTRR
and contiguous layouts, and matches the fp64 oracle on full shares."""
import dataclasses

import pytest
import torch

import block_sparse_masked_metadata_amd as bsm
from workloads import packed_multimodal, packed_text, sliding_window
from gpu_common import Case, check_rows, needs_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not needs_gpu, reason="needs a GPU")]


@pytest.mark.parametrize("make,order", [(packed_text, "ptrr"), (packed_text, "contiguous"),
                                        (packed_multimodal, "contiguous"), (sliding_window, "contiguous")])
def test_fetched_pass_equals_single_pass(make, order):
    lay = dataclasses.replace(make(), order=order)
    case = Case(lay)
    need, cnt = case.plan.fetch_set(case.r)
    assert case.dp.info["fetch_tiles"] == cnt
    assert case.dp.info["fetch_rows"] == case.S + 128 * cnt
    o1, lse1 = case.single()
    kf, vf = bsm.gather_fetched(case.plan, case.r, case.k_all, case.v_all)
    o2, lse2 = bsm.fwd_fetched(case.dp, case.heads, case.q, kf, vf)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(lse1, lse2)


@pytest.mark.parametrize("make,order", [(packed_text, "contiguous"), (packed_multimodal, "contiguous")])
def test_fetched_pass_matches_oracle(make, order):
    """The fetched pass against the oracle on the busiest contiguous rank's
    full share: O before rounding (its KEEP_STATE state) within 1e-2, bf16 O
    its round-to-nearest-even, LSE within 1e-3."""
    lay = dataclasses.replace(make(), order=order)
    case = Case(lay)
    kf, vf = bsm.gather_fetched(case.plan, case.r, case.k_all, case.v_all)
    o, lse = bsm.fwd_fetched(case.dp, case.heads, case.q, kf, vf)
    st = bsm.fwd_fetched(case.dp, case.heads, case.q, kf, vf, keep_state=True)
    torch.cuda.synchronize()
    check_rows(case, o, lse, state=st)
