"""Shared setup of the GPU parity tests: plan, device plan, seeded inputs in
plan order, and comparison helpers.  Inputs come from workloads/, expected
values from oracle/ only."""
import numpy as np
import torch

import block_sparse_masked_metadata_amd as bsm
from workloads import qkv

O_TOL = 1e-2      # max |O - O_ref| for bf16 inputs
LSE_TOL = 1e-3    # max |LSE - LSE_ref|
GRAD_REL = 1e-2   # max |g - g_ref| <= GRAD_REL * max(1, max |g_ref|)

needs_gpu = torch.cuda.is_available()


class Case:
    """One rank's share of a layout on the GPU."""

    def __init__(self, lay, rank=None, with_do=False, tensors=None, hq=None, hkv=None):
        self.lay = lay
        self.hq = hq or lay.hq
        self.hkv = hkv or lay.hkv
        self.d = 128
        self.plan = bsm.Plan.from_layout(lay)
        self.r = self.plan.info["busiest_rank"] if rank is None else rank
        self.dp = bsm.DevicePlan(self.plan, self.r)
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
