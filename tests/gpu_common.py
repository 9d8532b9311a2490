"""Shared setup of the GPU parity tests: plan, device plan, seeded inputs in
plan order, and comparison helpers.  Inputs come from workloads/, expected
values from oracle/ only."""
import numpy as np
import torch

import block_sparse_masked_metadata_amd as bsm
from workloads import qkv
from oracle import attention as oatt

O_TOL = 1e-2      # max |O - O_ref| for bf16 inputs
LSE_TOL = 1e-3    # max |LSE - LSE_ref|
GRAD_REL = 1e-2   # max |g - g_ref| <= GRAD_REL * max(1, max |g_ref|)

needs_gpu = torch.cuda.is_available()


class Case:
    """One rank's share of a layout on the GPU."""

    def __init__(self, lay, rank=None, with_do=False, tensors=None, hq=None, hkv=None, dense=False):
        self.lay = lay
        self.hq = hq or lay.hq
        self.hkv = hkv or lay.hkv
        self.d = 128
        self.plan = bsm.Plan.from_layout(lay)
        self.r = self.plan.info["busiest_rank"] if rank is None else rank
        self.dp = bsm.DevicePlan(self.plan, self.r, dense=dense)
        self.R = lay.ranks
        self.S = self.plan.info["shard_tokens"]
        self.perm = self.plan.permutation().astype(np.int64)
        self.rows = self.perm[self.r * self.S:(self.r + 1) * self.S]
        if tensors is None:
            tensors = qkv(lay.n, self.hq, self.hkv, self.d, lay.seed, "cuda", with_do=with_do)
        self.full = tensors                      # original order, on the GPU
        pidx = torch.from_numpy(self.perm).cuda()
        ridx = torch.from_numpy(self.rows).cuda()
        self.q = tensors[0][ridx].contiguous()
        self.k_all = tensors[1][pidx].contiguous()
        self.v_all = tensors[2][pidx].contiguous()
        self.dout = tensors[3][ridx].contiguous() if len(tensors) > 3 else None
        self.k_shards = [self.k_all[j * self.S:(j + 1) * self.S] for j in range(self.R)]
        self.v_shards = [self.v_all[j * self.S:(j + 1) * self.S] for j in range(self.R)]
        self.heads = bsm.heads(self.hq, self.hkv, self.d, 1.0 / np.sqrt(lay.d))

    def cpu(self, i):
        return self.full[i].cpu()

    def ring(self, **kw):
        return bsm.fwd_ring(self.dp, self.heads, self.q, self.k_shards, self.v_shards, **kw)

    def single(self, **kw):
        return bsm.fwd_single(self.dp, self.heads, self.q, self.k_all, self.v_all, **kw)


def max_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), "non-finite pattern differs"
    return float(np.abs(a[fin] - b[fin]).max()) if fin.any() else 0.0


def grad_ok(g, ref, name):
    tol = GRAD_REL * max(1.0, float(np.abs(ref).max()))
    err = float(np.abs(np.asarray(g, np.float64) - ref).max())
    assert err <= tol, f"{name}: max err {err:.3e} > {tol:.3e}"
    return err


def check_rows(case, o, lse, sel=None, tol_o=O_TOL, tol_lse=LSE_TOL, single=False, state=None):
    """Compare GPU rows (indices into the rank's shard) with the oracle.

    The O bar applies to the value the kernel rounds to bf16 (O_acc times the
    fp32 reciprocal of l, from a KEEP_STATE run of the same launches); the
    bf16 output must be exactly that value rounded to nearest even.  LSE is
    compared as written.  state: the KEEP_STATE (O_acc, m, l) of the launches
    that wrote o and lse, when neither the ring nor the single pass did."""
    sel = np.arange(case.S) if sel is None else np.asarray(sel)
    q, k, v = case.cpu(0), case.cpu(1), case.cpu(2)
    o_ref, lse_ref = oatt.forward_rows(case.lay.tracks(), case.lay.window, q, k, v,
                                       case.rows[sel], 1.0 / np.sqrt(case.lay.d))
    tsel = torch.from_numpy(sel).cuda()
    if state is None:
        state = case.single(keep_state=True) if single else case.ring(keep_state=True)[2]
    acc, m, l = state
    acc = bsm.state_rows(case.heads, acc, case.S)[tsel].cpu()
    l = l[:, tsel].cpu().T[:, :, None]
    rl = torch.where(l > 0, 1.0 / torch.where(l > 0, l, torch.ones_like(l)), torch.zeros_like(l))
    o32 = acc * rl
    og = o[tsel].cpu()
    assert torch.equal(og, o32.to(torch.bfloat16)), "bf16 O is not RNE(O_acc * (1 / l))"
    lg = lse[:, tsel].cpu().numpy()
    eo = max_err(o32.numpy(), o_ref)
    eob = max_err(og.float().numpy(), o_ref)
    el = max_err(lg, lse_ref)
    print(f"  rank={case.r} rows={len(sel)} max|dO32|={eo:.3e} max|dO_bf16|={eob:.3e} "
          f"max|dLSE|={el:.3e}", flush=True)
    assert eo <= tol_o and el <= tol_lse
    return eo, el
