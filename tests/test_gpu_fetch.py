"""Sparse fetch on the GPU (MARBLE section 04, "Sparse all-to-all and strategy
selection"): one pass over the rank's shard and its fetched remote tiles is
bitwise the single pass over all shards (same tiles, same order), on PTRR
and contiguous layouts."""
import dataclasses

import pytest
import torch

import block_sparse_masked_metadata_amd as bsm
from workloads import packed_multimodal, packed_text, sliding_window
from gpu_common import Case, needs_gpu

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
