"""bsm_bwd_step_noalloc (split dK/dV partial sums in the library's static
scratch) against bsm_bwd_step_ws (the same kernels with a caller workspace):
bit-identical gradients on two calls in a row, the second with a smaller
input, through the C ABI.  Packed text is the workload whose steps split."""
import numpy as np
import pytest
import torch

import block_sparse_masked_metadata_amd as bsm
from block_sparse_masked_metadata_amd import _capi as C
from workloads import packed_text
from gpu_common import Case, needs_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not needs_gpu, reason="needs a GPU")]

SCRATCH_BYTES = 64 << 20


def _grads(case, o, lse, delta, call):
    dq = torch.full((case.S, case.hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    dks = [torch.zeros(case.S, case.hkv, 128, dtype=torch.float32, device="cuda") for _ in range(case.R)]
    dvs = [torch.zeros_like(t) for t in dks]
    st = torch.cuda.current_stream().cuda_stream
    for s in range(case.R):
        j = (case.r - s) % case.R
        args = (case.dp.handle, s, case.heads, case.q.data_ptr(), case.k_shards[j].data_ptr(),
                case.v_shards[j].data_ptr(), case.dout.data_ptr(), lse.data_ptr(), delta.data_ptr(),
                dq.data_ptr(), dks[j].data_ptr(), dvs[j].data_ptr())
        call(args, st)
    torch.cuda.synchronize()
    return [dq] + dks + dvs


def _check(lay):
    case = Case(lay, with_do=True)
    slots = case.dp.info["bwd_workspace_slots"]
    need = slots * case.hkv * 2 * 128 * 128 * 4
    print(f"  {lay.name} n={lay.n}: {slots} workspace slots, {need} bytes", flush=True)
    assert 0 < need <= SCRATCH_BYTES
    o, lse, _ = case.ring()
    delta = bsm.bwd_prep(case.heads, o, case.dout)
    ws = bsm.bwd_workspace(case.dp, case.heads)
    nbytes = ws.numel() * ws.element_size()
    want = _grads(case, o, lse, delta,
                  lambda a, st: C.bsm_bwd_step_ws(*a, ws.data_ptr(), nbytes, st))
    got = _grads(case, o, lse, delta, lambda a, st: C.bsm_bwd_step_noalloc(*a, st))
    for x, y in zip(got, want):
        assert torch.equal(x, y)
    # the split really ran: the unsplit call rounds the dK/dV sums differently
    plain = _grads(case, o, lse, delta, lambda a, st: C.bsm_bwd_step(*a, st))
    assert any(not torch.equal(x, y) for x, y in zip(got[1:], plain[1:]))
    return need


def test_noalloc_matches_workspace_entry_point():
    big = _check(packed_text())
    small = _check(packed_text(n=16384, seed=7))
    assert small < big
