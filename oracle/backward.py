"""Gradients of masked softmax attention, fp64, per sample.

MARBLE (section 03, "Exact ring attention accumulation") runs a FlashAttention
backward per ring step against the final LSE, carries an fp32 dQ accumulator
across steps and lets each shard's fp32 dK/dV accumulator travel; the pages do
not write the gradient out.  The result it reaches is the ordinary derivative
of O = softmax(scale * Q K^T + M) V, written here from that definition:
    P_ij  = exp(s_ij - LSE_i)              on legal pairs, 0 elsewhere
    D_i   = sum_c dO_ic O_ic
    dV_j  = sum_i P_ij dO_i
    dP_ij = dO_i . v_j
    dS_ij = P_ij (dP_ij - D_i)
    dQ_i  = scale * sum_j dS_ij k_j
    dK_j  = scale * sum_i dS_ij q_i
With grouped-query attention dK and dV of a key/value head sum over the query
heads of its group.  For one rank's share only that rank's query rows
contribute to dK/dV.

The dense products and elementwise steps run as torch CPU ops in fp64
(threaded GEMM and exp), one (query head) at a time.  Query rows are taken in
chunks; each chunk is evaluated against the keys legal for at least one of its
rows only.  That restriction is exact: a key no row of the chunk may read has
P = 0 for all of them and so adds nothing to O, l, dQ, dK or dV of the chunk.

Pinned by: tests/test_oracle_backward.py (central finite differences of
L = sum(dO * O) in fp64 on tiny masked layouts, with chunks smaller than the
row set; dK/dV vanish on keys no query of the share may read; the key-sum
identities).
"""
from __future__ import annotations

import numpy as np

from .attention import as_f64, gather, kv_head, sample_ranges
from .mask import legal, take


def attention_grads_fp64(q, k, v, do, allowed, scale: float):
    """Dense per-block gradients.

    q, do [nq, Hq, d]; k, v [nk, Hkv, d]; allowed [nq, nk] (bool).
    Returns O, LSE, D, dQ, dK, dV (fp64 numpy arrays).
    """
    import torch
    f64 = torch.float64
    q, k, v, do = (torch.from_numpy(np.ascontiguousarray(as_f64(x))) for x in (q, k, v, do))
    allowed = torch.from_numpy(np.ascontiguousarray(allowed, bool))
    nq, hq, d = q.shape
    nk, hkv, _ = k.shape
    o = torch.zeros(nq, hq, v.shape[2], dtype=f64)
    lse = torch.full((hq, nq), -np.inf, dtype=f64)
    dlt = torch.zeros(hq, nq, dtype=f64)
    dq = torch.zeros_like(q)
    dk = torch.zeros_like(k)
    dv = torch.zeros_like(v)
    any_legal = allowed.any(dim=1)
    if nk == 0 or not bool(any_legal.any()):
        return o.numpy(), lse.numpy(), dlt.numpy(), dq.numpy(), dk.numpy(), dv.numpy()
    zero = torch.zeros((), dtype=f64)
    for h in range(hq):
        g = kv_head(h, hq, hkv)
        qh, doh = q[:, h, :].contiguous(), do[:, h, :].contiguous()
        kg, vg = k[:, g, :].contiguous(), v[:, g, :].contiguous()
        s = qh @ kg.T                                          # s_ij / scale
        s.mul_(scale).masked_fill_(~allowed, -np.inf)          # s_ij, -inf on illegal pairs
        m = torch.where(any_legal, s.amax(dim=1), zero)        # row max (0 for empty rows)
        p = s.sub_(m[:, None]).exp_()                          # e^(s_ij - m_i), 0 where illegal
        l = p.sum(dim=1)
        lse_h = torch.where(any_legal, m + torch.log(torch.where(l > 0, l, torch.ones_like(l))),
                            torch.full_like(l, -np.inf))
        p.div_(torch.where(l > 0, l, torch.ones_like(l))[:, None])   # P_ij = e^(s_ij - LSE_i)
        oh = p @ vg                                            # O_i
        dh = (doh * oh).sum(dim=1)                             # D_i
        ds = (doh @ vg.T).sub_(dh[:, None]).mul_(p)            # dS_ij = P_ij (dO_i . v_j - D_i)
        o[:, h, :] = oh
        lse[h] = lse_h
        dlt[h] = dh
        dq[:, h, :] = scale * (ds @ kg)
        dk[:, g, :] += scale * (ds.T @ qh)
        dv[:, g, :] += p.T @ doh
    return o.numpy(), lse.numpy(), dlt.numpy(), dq.numpy(), dk.numpy(), dv.numpy()


def backward_rows(tracks, window: int, q, k, v, do, rows, scale: float, chunk: int = 512):
    """Gradients of the share whose query tokens are `rows` (original indices).

    Returns dict with o, lse, delta, dq (in the order of `rows`) and `dkv`:
    a list of (key_start, key_end, dk, dv) per sample touched, keys in the
    original order.  Rows are evaluated `chunk` at a time, each chunk against
    the keys of its sample that at least one of its rows may read.
    """
    rows = np.asarray(rows, np.int64)
    sample = np.asarray(tracks[0])
    ranges = sample_ranges(sample)
    hq = q.shape[1]
    hkv = k.shape[1]
    d = q.shape[2]
    out = {
        "o": np.zeros((len(rows), hq, d)),
        "lse": np.full((hq, len(rows)), -np.inf),
        "delta": np.zeros((hq, len(rows))),
        "dq": np.zeros((len(rows), hq, d)),
        "dkv": [],
    }
    by_sample = {}
    for i, t in enumerate(rows):
        by_sample.setdefault(int(sample[t]), []).append(i)
    for sid in sorted(by_sample):
        idx = np.asarray(by_sample[sid])
        a, b = ranges[sid]
        kt = take(tracks, np.arange(a, b))
        dk = np.zeros((b - a, hkv, d))
        dv = np.zeros((b - a, hkv, d))
        for c0 in range(0, len(idx), chunk):
            part = idx[c0:c0 + chunk]
            allowed = legal(take(tracks, rows[part]), kt, window)
            cols = np.flatnonzero(allowed.any(axis=0))     # keys some row of the chunk reads
            o, lse, dl, dq, dkc, dvc = attention_grads_fp64(
                gather(q, rows[part]), gather(k, a + cols), gather(v, a + cols),
                gather(do, rows[part]), allowed[:, cols], scale)
            out["o"][part] = o
            out["lse"][:, part] = lse
            out["delta"][:, part] = dl
            out["dq"][part] = dq
            dk[cols] += dkc
            dv[cols] += dvc
        out["dkv"].append((a, b, dk, dv))
    return out
