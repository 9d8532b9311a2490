"""GPU parity on chunked ring layouts and of the dense-call mode (MARBLE
section 03, "Chunked ring attention"): each rank owns k contiguous chunks
chosen by the planner's search, and each ring step can run as dense calls;
every rank's ring steps must still match the fp64 oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import block_sparse_masked_metadata_amd as bsm
from workloads import random_small, packed_multimodal, long_mixed, packed_text
from gpu_common import Case, check_rows, needs_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not needs_gpu, reason="needs a GPU")]


def _chunked(lay, min_chunks, max_chunks, tau=0.0, swaps=2):
    base = bsm.Plan.from_layout(dataclasses.replace(lay, order="contiguous"))
    perm, info = base.chunk_order(min_chunks, max_chunks, tau, swaps)
    return dataclasses.replace(lay, order="explicit", block_perm=perm), info


def _check(case, sel, single=False):
    o, lse = case.single() if single else case.ring()[:2]
    torch.cuda.synchronize()
    check_rows(case, o, lse, sel, single=single)


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


@pytest.mark.parametrize("seed", range(6))
def test_dense_calls_random_every_rank(seed):
    """All five span modes, noise spans and finite windows, every rank."""
    rng = np.random.default_rng(1300 + seed)
    R = [1, 2, 4, 3, 2, 4][seed]
    lay = random_small(rng, 128 * R * [2, 3, 1, 2, 4, 2][seed], max_span=[300, 40, 500, 120, 60, 900][seed])
    lay.ranks, lay.seed = R, 80 + seed
    lay.order = ["ptrr", "contiguous"][seed % 2]
    lay.hq, lay.hkv = [(4, 2), (2, 1), (8, 8), (4, 1), (6, 2), (2, 2)][seed]
    lay.d = 128
    print(f"  window={lay.window} order={lay.order}", flush=True)
    for r in range(R):
        case = Case(lay, rank=r, dense=True)
        assert case.dp.info["dense_calls"]
        _check(case, np.arange(case.S))


def test_dense_calls_single_pass_matches_oracle():
    rng = np.random.default_rng(1400)
    lay = random_small(rng, 128 * 3 * 2, max_span=200)
    lay.ranks, lay.seed, lay.order = 3, 91, "ptrr"
    lay.hq, lay.hkv, lay.d = 4, 2, 128
    for r in range(3):
        _check(Case(lay, rank=r, dense=True), np.arange(128 * 2), single=True)


def test_dense_calls_packed_text_full_share():
    case = Case(packed_text(), dense=True)
    _check(case, np.arange(case.S))


def test_dense_calls_long_mixed_chunked_sampled():
    lay, info = _chunked(long_mixed(), 1, 8)
    case = Case(lay, dense=True)
    rng = np.random.default_rng(4)
    _check(case, np.sort(rng.choice(case.S, 256, replace=False)))


def test_dense_calls_refuse_fetch():
    case = Case(packed_text(), dense=True)
    C = bsm._capi
    z = case.q.data_ptr()
    with pytest.raises(bsm.BsmError) as e:
        C.bsm_fwd_fetched(case.dp.handle, case.heads, z, z, z, None, None, None, z, z, 0, None)
    assert e.value.code == C.BSM_E_UNSUPPORTED


def _grads(case):
    o, lse, _ = case.ring()
    dq, dks, dvs = bsm.bwd_ring(case.dp, case.heads, case.q, case.k_shards, case.v_shards,
                                case.dout, o, lse)
    torch.cuda.synchronize()
    return dq, dks, dvs


@pytest.mark.parametrize("seed", range(4))
def test_dense_calls_backward_matches_oracle(seed):
    """Dense-call backward lists (row pieces for dQ, key-tile column pieces for
    dK/dV): every rank's gradients against the fp64 oracle."""
    from oracle import backward as obwd
    from gpu_common import grad_ok
    rng = np.random.default_rng(1600 + seed)
    R = [2, 3, 1, 4][seed]
    lay = random_small(rng, 128 * R * [2, 2, 3, 1][seed], max_span=[300, 60, 700, 150][seed])
    lay.ranks, lay.seed = R, 95 + seed
    lay.order = ["ptrr", "contiguous"][seed % 2]
    lay.hq, lay.hkv = [(4, 2), (2, 1), (4, 4), (6, 3)][seed]
    lay.d = 128
    print(f"  window={lay.window} order={lay.order}", flush=True)
    for r in range(R):
        case = Case(lay, rank=r, with_do=True, dense=True)
        dq, dks, dvs = _grads(case)
        ref = obwd.backward_rows(lay.tracks(), lay.window, case.cpu(0), case.cpu(1), case.cpu(2),
                                 case.cpu(3), case.rows, 1.0 / np.sqrt(lay.d))
        e1 = grad_ok(dq.cpu().numpy(), ref["dq"], "dq")
        dk = np.zeros((lay.n, lay.hkv, 128))
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
        print(f"  rank={r} dq {e1:.3e} dk {e2:.3e} dv {e3:.3e}", flush=True)


def test_dense_calls_backward_equals_block_sparse_closely():
    """Same share, both list kinds: gradients agree to accumulation-order rounding."""
    lay = packed_text()
    a = Case(lay, with_do=True)
    b = Case(lay, with_do=True, tensors=a.full, dense=True)
    ga, gb = _grads(a), _grads(b)
    for x, y in zip([ga[0]] + list(ga[1]) + list(ga[2]), [gb[0]] + list(gb[1]) + list(gb[2])):
        scale = max(1.0, float(x.abs().max()))
        assert float((x - y).abs().max()) <= 2e-3 * scale


@pytest.mark.parametrize("dense", [False, True], ids=["block_sparse", "dense_calls"])
@pytest.mark.parametrize("R,S", [(2, 200), (3, 330)])
def test_ragged_shards_forward_backward(R, S, dense):
    """Contiguous shards of S tokens (S not a multiple of 128): a ragged last
    query and key tile, the padded tile-blocked state, every rank, forward
    and backward against the oracle."""
    from oracle import backward as obwd
    from gpu_common import grad_ok
    rng = np.random.default_rng(1700 + S + R)
    lay = random_small(rng, R * S, max_span=150)
    lay.ranks, lay.order, lay.seed = R, "contiguous", 120 + S
    lay.hq, lay.hkv, lay.d = 4, 2, 128
    for r in range(R):
        case = Case(lay, rank=r, with_do=True, dense=dense)
        assert case.S == S
        _check(case, np.arange(S))
        dq, dks, dvs = _grads(case)
        ref = obwd.backward_rows(lay.tracks(), lay.window, case.cpu(0), case.cpu(1), case.cpu(2),
                                 case.cpu(3), case.rows, 1.0 / np.sqrt(lay.d))
        grad_ok(dq.cpu().numpy(), ref["dq"], "dq")
        dk = np.zeros((lay.n, lay.hkv, 128))
        dv = np.zeros_like(dk)
        dk[case.perm] = torch.cat(dks).cpu().numpy()
        dv[case.perm] = torch.cat(dvs).cpu().numpy()
        dk_ref = np.zeros_like(dk)
        dv_ref = np.zeros_like(dv)
        for a, b, dkb, dvb in ref["dkv"]:
            dk_ref[a:b] += dkb
            dv_ref[a:b] += dvb
        grad_ok(dk, dk_ref, "dk")
        grad_ok(dv, dv_ref, "dv")
