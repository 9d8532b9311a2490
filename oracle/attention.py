"""Masked softmax attention from its definition, fp64, per sample.

Definition (ring-attention explainer, "The Long-Context Scaling Problem":
Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V; Libra page, section 2.2,
Eq. 1, with an additive mask M in {0, -inf}).  For query row i and head h:
    s_ij   = scale * sum_c q_ic k_jc            over keys j legal for i
    m_i    = max_j s_ij
    l_i    = sum_j exp(s_ij - m_i)
    O_i    = sum_j exp(s_ij - m_i) v_j / l_i
    LSE_i  = m_i + ln l_i
A row with no legal key has l_i = 0; it is defined here as O_i = 0 and
LSE_i = -inf (never reached by a full share: every token sees itself).

Grouped-query attention: query head h reads key/value head floor(h / (Hq/Hkv))
(contiguous groups; the pages do not fix the head map).

Because same_sample is one factor of the mask (MARBLE, section 01), attention
of any set of query rows decomposes exactly into independent per-sample
problems; `forward_rows` uses that to evaluate only a sample's own keys.

Pinned by: tests/test_oracle_attention.py (softmax rows sum to 1; zero weight
across samples; Q = 0 gives LSE = ln(#legal keys) with the count from the
layout's closed form; V = 1 gives O = 1; a dense unmasked case reproduces
torch's scaled_dot_product_attention on the CPU; permutation invariance).
"""
from __future__ import annotations

import numpy as np

from .mask import legal, take


def as_f64(x) -> np.ndarray:
    """Accept numpy or torch (any float dtype, incl. bfloat16) and return fp64."""
    if hasattr(x, "detach"):
        import torch
        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def gather(x, idx):
    """Rows `idx` of a numpy or torch array, as an fp64 numpy array."""
    idx = np.asarray(idx, np.int64)
    if hasattr(x, "detach"):
        import torch
        return as_f64(x[torch.from_numpy(idx)])
    return as_f64(np.asarray(x)[idx])


def kv_head(h: int, hq: int, hkv: int) -> int:
    return h // (hq // hkv)


def attention_fp64(q, k, v, allowed, scale: float):
    """q [nq, Hq, d], k/v [nk, Hkv, d], allowed [nq, nk] -> (O [nq,Hq,d], LSE [Hq,nq])."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    nq, hq, d = q.shape
    hkv = k.shape[1]
    out = np.zeros((nq, hq, v.shape[2]), np.float64)
    lse = np.full((hq, nq), -np.inf, np.float64)
    any_legal = allowed.any(axis=1)
    for h in range(hq):
        g = kv_head(h, hq, hkv)
        s = scale * (q[:, h, :] @ k[:, g, :].T)
        s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1) if s.shape[1] else np.full(nq, -np.inf)
        m_safe = np.where(any_legal, m, 0.0)
        e = np.exp(s - m_safe[:, None])
        l = e.sum(axis=1)
        with np.errstate(invalid="ignore", divide="ignore"):
            out[:, h, :] = np.where(any_legal[:, None], (e @ v[:, g, :]) / l[:, None], 0.0)
            lse[h] = np.where(any_legal, m + np.log(l), -np.inf)
    return out, lse


def sample_ranges(sample: np.ndarray):
    """Map sample id -> [start, end) in the original order (samples are contiguous runs)."""
    sample = np.asarray(sample)
    change = np.flatnonzero(np.diff(sample)) + 1
    starts = np.concatenate([[0], change])
    ends = np.concatenate([change, [len(sample)]])
    return {int(sample[a]): (int(a), int(b)) for a, b in zip(starts, ends)}


def forward_rows(tracks, window: int, q, k, v, rows, scale: float, chunk: int = 4096):
    """O and LSE of the query tokens `rows` (original indices), keys = all tokens.

    q, k, v are full original-order arrays.  Returns O [len(rows), Hq, d] and
    LSE [Hq, len(rows)] in the order of `rows`.
    """
    rows = np.asarray(rows, np.int64)
    sample = np.asarray(tracks[0])
    ranges = sample_ranges(sample)
    hq = q.shape[1]
    o = np.zeros((len(rows), hq, v.shape[2]), np.float64)
    lse = np.full((hq, len(rows)), -np.inf, np.float64)
    by_sample = {}
    for i, t in enumerate(rows):
        by_sample.setdefault(int(sample[t]), []).append(i)
    for sid, idx in by_sample.items():
        a, b = ranges[sid]
        keys = np.arange(a, b)
        kt = take(tracks, keys)
        idx = np.asarray(idx)
        kk, vv = as_f64(k[a:b]), as_f64(v[a:b])
        for c0 in range(0, len(idx), chunk):
            part = idx[c0:c0 + chunk]
            allowed = legal(take(tracks, rows[part]), kt, window)
            oo, ll = attention_fp64(gather(q, rows[part]), kk, vv, allowed, scale)
            o[part] = oo
            lse[:, part] = ll
    return o, lse


def legal_counts(tracks, window: int, rows):
    """Number of legal keys of each query in `rows` (original indices), from the mask."""
    rows = np.asarray(rows, np.int64)
    sample = np.asarray(tracks[0])
    ranges = sample_ranges(sample)
    out = np.zeros(len(rows), np.int64)
    for i, t in enumerate(rows):
        a, b = ranges[int(sample[t])]
        out[i] = legal(take(tracks, [t]), take(tracks, np.arange(a, b)), window).sum()
    return out
