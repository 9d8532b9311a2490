"""GPU parity on chunked ring layouts (MARBLE section 03, "Chunked ring
attention"): each rank owns k contiguous chunks chosen by the planner's
search; every rank's ring steps must still match the fp64 oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import block_sparse_masked_metadata_amd as bsm
from workloads import random_small, packed_multimodal
from oracle import attention as oatt
from gpu_common import Case, O_TOL, LSE_TOL, max_err, needs_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not needs_gpu, reason="needs a GPU")]


def _chunked(lay, min_chunks, max_chunks, tau=0.0, swaps=2):
    base = bsm.Plan.from_layout(dataclasses.replace(lay, order="contiguous"))
    perm, info = base.chunk_order(min_chunks, max_chunks, tau, swaps)
    return dataclasses.replace(lay, order="explicit", block_perm=perm), info


def _check(case, sel):
    o, lse, _ = case.ring()
    torch.cuda.synchronize()
    o_ref, lse_ref = oatt.forward_rows(case.lay.tracks(), case.lay.window, case.cpu(0),
                                       case.cpu(1), case.cpu(2), case.rows[sel],
                                       1.0 / np.sqrt(case.lay.d))
    tsel = torch.from_numpy(sel).cuda()
    eo = max_err(o[tsel].float().cpu().numpy(), o_ref)
    el = max_err(lse[:, tsel].cpu().numpy(), lse_ref)
    print(f"  rank={case.r} rows={len(sel)} max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL and el <= LSE_TOL


@pytest.mark.parametrize("seed", range(3))
def test_chunked_random_every_rank(seed):
    rng = np.random.default_rng(1200 + seed)
    R = [4, 2, 3][seed]
    lay = random_small(rng, 128 * R * 4, max_span=400)
    lay.ranks, lay.seed, lay.block = R, 60 + seed, 128
    lay.hq, lay.hkv, lay.d = 4, 2, 128
    lay, info = _chunked(lay, 2, 4)
    print(f"  chunks_per_rank={info['chunks_per_rank']} strategy={info['strategy']}", flush=True)
    for r in range(R):
        case = Case(lay, rank=r)
        _check(case, np.arange(case.S))


def test_chunked_packed_multimodal_sampled():
    lay, info = _chunked(packed_multimodal(), 1, 16)
    print(f"  chunks_per_rank={info['chunks_per_rank']} strategy={info['strategy']} "
          f"cost={info['cost']:.0f}", flush=True)
    case = Case(lay)
    rng = np.random.default_rng(3)
    _check(case, np.sort(rng.choice(case.S, 512, replace=False)))
