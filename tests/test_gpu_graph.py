"""The ring forward and backward captured in a HIP graph (torch.cuda.CUDAGraph
over the library's launches on the current stream and the two side streams):
every replay gives the eager results bit for bit, with eager work, poisoned
outputs and synchronizations between the replays."""
import numpy as np
import pytest
import torch

import block_sparse_masked_metadata_amd as bsm
from workloads import random_small, packed_multimodal, packed_text
from gpu_common import Case, needs_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not needs_gpu, reason="needs a GPU")]


def _random(seed):
    rng = np.random.default_rng(seed)
    lay = random_small(rng, 128 * 4 * 4, max_span=300)
    lay.ranks, lay.order, lay.seed = 4, "ptrr", seed
    lay.hq, lay.hkv, lay.d = 4, 2, 128
    return lay


def _pass(case, st, out, grads):
    o, lse, _ = case.ring(state=st, out=out)
    bsm.bwd_ring(case.dp, case.heads, case.q, case.k_shards, case.v_shards, case.dout, o, lse, grads=grads)


@pytest.mark.parametrize("maker", ["packed_multimodal", "packed_text", "random5"])
def test_graph_replays_equal_eager(maker):
    lay = {"packed_multimodal": packed_multimodal, "packed_text": packed_text}.get(maker)
    lay = lay() if lay else _random(5)
    case = Case(lay, with_do=True)
    o_e, lse_e, _ = case.ring()
    dq_e, dks_e, dvs_e = bsm.bwd_ring(case.dp, case.heads, case.q, case.k_shards, case.v_shards, case.dout,
                                      o_e, lse_e)
    torch.cuda.synchronize()

    st = bsm.new_state(case.S, case.hq, 128)
    out = (torch.empty_like(o_e), torch.empty_like(lse_e))
    grads = (torch.empty_like(dq_e), [torch.empty_like(t) for t in dks_e], [torch.empty_like(t) for t in dvs_e])
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        for _ in range(2):
            _pass(case, st, out, grads)
    torch.cuda.current_stream().wait_stream(warm)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _pass(case, st, out, grads)
    torch.cuda.synchronize()

    for rep in range(3):
        for t in (out[0], out[1], grads[0], *grads[1], *grads[2]):
            t.fill_(float("nan"))
        case.ring()  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out[0], o_e) and torch.equal(out[1], lse_e), f"replay {rep}: O/LSE"
        assert torch.equal(grads[0], dq_e), f"replay {rep}: dQ"
        for a, b in zip(grads[1] + grads[2], dks_e + dvs_e):
            assert torch.equal(a, b), f"replay {rep}: dK/dV"
