"""Sparse fetch on the GPU (MARBLE section 04, "Sparse all-to-all and strategy
selection"): one pass over the rank's shard and its fetched remote tiles is
bitwise the single pass over all shards (same tiles, same order), on PTRR
and contiguous layouts, and matches the fp64 oracle on full shares; its
backward (dQ, and dK/dV of the fetched tiles sent back to their shards)
matches the oracle and the ring backward."""
import dataclasses

import numpy as np
import pytest
import torch

import block_sparse_masked_metadata_amd as bsm
from workloads import packed_multimodal, packed_text, sliding_window, random_small
from oracle import backward as obwd
from gpu_common import Case, check_rows, grad_ok, needs_gpu

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


def _fetched_grads(case):
    """Fetched forward and backward of the case's rank, the compact dK/dV sent
    back to the shards; returns (o, lse, dq, dk_all, dv_all) with dk/dv over
    all shards in plan order."""
    kf, vf = bsm.gather_fetched(case.plan, case.r, case.k_all, case.v_all)
    o, lse = bsm.fwd_fetched(case.dp, case.heads, case.q, kf, vf)
    dq, dkf, dvf = bsm.bwd_fetched(case.dp, case.heads, case.q, kf, vf, case.dout, o, lse)
    dk_all = torch.zeros(case.R * case.S, case.hkv, 128, dtype=torch.float32, device="cuda")
    dv_all = torch.zeros_like(dk_all)
    bsm.fetched_accumulate(case.dp, case.heads, dkf, dvf, dk_all, dv_all)
    torch.cuda.synchronize()
    return o, lse, dq, dk_all, dv_all


def _check_grads(case, dq, dk_all, dv_all):
    ref = obwd.backward_rows(case.lay.tracks(), case.lay.window, case.cpu(0), case.cpu(1), case.cpu(2),
                             case.cpu(3), case.rows, 1.0 / np.sqrt(case.lay.d))
    e1 = grad_ok(dq.cpu().numpy(), ref["dq"], "dq")
    n = case.lay.n
    dk = np.zeros((n, case.hkv, 128))
    dv = np.zeros_like(dk)
    dk[case.perm] = dk_all.cpu().numpy()
    dv[case.perm] = dv_all.cpu().numpy()
    dk_ref = np.zeros_like(dk)
    dv_ref = np.zeros_like(dv)
    for a, b, dkb, dvb in ref["dkv"]:
        dk_ref[a:b] += dkb
        dv_ref[a:b] += dvb
    e2 = grad_ok(dk, dk_ref, "dk")
    e3 = grad_ok(dv, dv_ref, "dv")
    print(f"  rank={case.r} fetched backward: dq {e1:.3e} dk {e2:.3e} dv {e3:.3e}", flush=True)


@pytest.mark.parametrize("make", [packed_text, packed_multimodal])
def test_fetched_backward_matches_oracle_and_ring(make):
    """MARBLE section 04: the fetched pass's dQ, and dK/dV of the fetched
    tiles returned to their shards, against the oracle on the busiest
    contiguous rank's full share, and against the ring backward of the same
    layout (equal up to the order of the fp32 sums)."""
    lay = dataclasses.replace(make(), order="contiguous")
    case = Case(lay, with_do=True)
    o, lse, dq, dk_all, dv_all = _fetched_grads(case)
    _check_grads(case, dq, dk_all, dv_all)
    o_r, lse_r, _ = case.ring()
    assert torch.equal(o, o_r) and torch.equal(lse, lse_r)
    g = bsm.bwd_ring(case.dp, case.heads, case.q, case.k_shards, case.v_shards, case.dout, o_r, lse_r)
    torch.cuda.synchronize()
    for x, y in ((dq, g[0]), (dk_all, torch.cat(g[1])), (dv_all, torch.cat(g[2]))):
        assert float((x - y).abs().max()) <= 1e-3 * max(1.0, float(y.abs().max()))


@pytest.mark.parametrize("seed", range(2))
def test_fetched_backward_ragged_every_rank(seed):
    """Contiguous shards of 330 tokens (tiles of 128, 128 and 74 rows): a
    needed remote tile can be the ragged one, in the middle of the compact
    buffer.  Forward and backward of the fetched pass against the oracle at
    every rank."""
    rng = np.random.default_rng(1300 + seed)
    ranks = [3, 4][seed]
    lay = random_small(rng, 330 * ranks, max_span=260)
    lay.ranks, lay.order, lay.seed = ranks, "contiguous", 80 + seed
    lay.hq, lay.hkv, lay.d = [(4, 2), (2, 1)][seed] + (128,)
    for r in range(ranks):
        case = Case(lay, rank=r, with_do=True)
        o, lse, dq, dk_all, dv_all = _fetched_grads(case)
        st = bsm.fwd_fetched(case.dp, case.heads, case.q, *bsm.gather_fetched(case.plan, r, case.k_all, case.v_all),
                             keep_state=True)
        torch.cuda.synchronize()
        check_rows(case, o, lse, state=st)
        _check_grads(case, dq, dk_all, dv_all)
