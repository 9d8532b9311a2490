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

Pinned by: tests/test_oracle_backward.py (central finite differences of
L = sum(dO * O) in fp64 on tiny masked layouts; dK/dV vanish on keys no query
of the share may read).
"""
from __future__ import annotations

import numpy as np

from .attention import as_f64, gather, kv_head, sample_ranges
from .mask import legal, take


def attention_grads_fp64(q, k, v, do, allowed, scale: float):
    """Dense per-block gradients.

    q, do [nq, Hq, d]; k, v [nk, Hkv, d]; allowed [nq, nk].
    Returns O, LSE, D, dQ, dK, dV (fp64).
    """
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    nq, hq, d = q.shape
    nk, hkv, _ = k.shape
    o = np.zeros_like(q)
    lse = np.full((hq, nq), -np.inf)
    dlt = np.zeros((hq, nq))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    any_legal = allowed.any(axis=1)
    for h in range(hq):
        g = kv_head(h, hq, hkv)
        s = scale * (q[:, h, :] @ k[:, g, :].T)
        s = np.where(allowed, s, -np.inf)
        m = np.where(any_legal, s.max(axis=1) if nk else 0.0, 0.0)
        l = np.exp(s - m[:, None]).sum(axis=1)
        with np.errstate(divide="ignore"):
            lse_h = np.where(any_legal, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
        p = np.where(allowed, np.exp(s - np.where(any_legal, lse_h, 0.0)[:, None]), 0.0)
        oh = p @ v[:, g, :]
        dh = (do[:, h, :] * oh).sum(axis=1)
        dp = do[:, h, :] @ v[:, g, :].T
        ds = p * (dp - dh[:, None])
        o[:, h, :] = oh
        lse[h] = lse_h
        dlt[h] = dh
        dq[:, h, :] = scale * (ds @ k[:, g, :])
        dk[:, g, :] += scale * (ds.T @ q[:, h, :])
        dv[:, g, :] += p.T @ do[:, h, :]
    return o, lse, dlt, dq, dk, dv


def backward_rows(tracks, window: int, q, k, v, do, rows, scale: float):
    """Gradients of the share whose query tokens are `rows` (original indices).

    Returns dict with o, lse, delta, dq (in the order of `rows`) and `dkv`:
    a list of (key_start, key_end, dk, dv) per sample touched, keys in the
    original order.
    """
    rows = np.asarray(rows, np.int64)
    sample = np.asarray(tracks[0])
    ranges = sample_ranges(sample)
    hq = q.shape[1]
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
        allowed = legal(take(tracks, rows[idx]), take(tracks, np.arange(a, b)), window)
        o, lse, dl, dq, dk, dv = attention_grads_fp64(
            gather(q, rows[idx]), as_f64(k[a:b]), as_f64(v[a:b]), gather(do, rows[idx]),
            allowed, scale)
        out["o"][idx] = o
        out["lse"][:, idx] = lse
        out["delta"][:, idx] = dl
        out["dq"][idx] = dq
        out["dkv"].append((a, b, dk, dv))
    return out
