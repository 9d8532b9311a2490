"""GPU parity on layouts in vision-group order (MARBLE section 04, "Layout
transforms"): positions no longer rise with the token index, and partial
tiles test key intervals in the index coordinate.  Forward and backward
against the fp64 oracle, and the ring against the single pass bit for bit."""
import numpy as np
import pytest
import torch

import block_sparse_masked_metadata_amd as bsm
from workloads import random_small, video_group, permuted
from oracle import backward as obwd
from gpu_common import Case, check_rows, grad_ok, needs_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not needs_gpu, reason="needs a GPU")]


def _check(case):
    o, lse, _ = case.ring()
    o1, l1 = case.single()
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(lse, l1)
    check_rows(case, o, lse)
    dq, dks, dvs = bsm.bwd_ring(case.dp, case.heads, case.q, case.k_shards, case.v_shards, case.dout, o, lse)
    torch.cuda.synchronize()
    ref = obwd.backward_rows(case.lay.tracks(), case.lay.window, case.cpu(0), case.cpu(1), case.cpu(2),
                             case.cpu(3), case.rows, 1.0 / np.sqrt(case.lay.d))
    e1 = grad_ok(dq.cpu().numpy(), ref["dq"], "dq")
    dk = np.zeros((case.lay.n, case.hkv, 128))
    dv = np.zeros_like(dk)
    dk[case.perm] = torch.cat(dks).cpu().numpy()
    dv[case.perm] = torch.cat(dvs).cpu().numpy()
    dk_ref = np.zeros_like(dk)
    dv_ref = np.zeros_like(dv)
    for a, b, dkb, dvb in ref["dkv"]:
        dk_ref[a:b] += dkb
        dv_ref[a:b] += dvb
    e2 = grad_ok(dk, dk_ref, "dk")
    e3 = grad_ok(dv, dv_ref, "dv")
    print(f"  rank={case.r} dq {e1:.3e} dk {e2:.3e} dv {e3:.3e}", flush=True)


def test_video_vision_group_full_share():
    lay = video_group()
    lay_v = permuted(lay, bsm.vision_group_order(lay.tracks()), name="video_group_128k_vision")
    case = Case(lay_v, with_do=True)
    assert case.plan.info["interval_keys"] == lay.n
    _check(case)


@pytest.mark.parametrize("seed", range(3))
def test_random_vision_group_every_rank(seed):
    rng = np.random.default_rng(2300 + seed)
    ranks = [2, 4, 3][seed]
    order = ["ptrr", "contiguous", "ptrr"][seed]
    base = random_small(rng, 128 * ranks * 2, max_span=200)
    lay = permuted(base, bsm.vision_group_order(base.tracks()))
    lay.ranks, lay.order, lay.seed = ranks, order, 90 + seed
    lay.hq, lay.hkv, lay.d = [(4, 2), (2, 2), (4, 1)][seed] + (128,)
    for r in range(ranks):
        _check(Case(lay, rank=r, with_do=True))
