"""The packed-mask predicate over the four metadata tracks.

MARBLE page, section "01 Packed multimodal masks", the mask code block: a query
q may attend a key k iff
    (causal(q,k) or same_span(q,k)) and keep_noise(q,k) and same_sample(q,k)
with
    causal(q,k)      : 0 <= pos[q] - pos[k] < W
    same_span(q,k)   : seg[q] == seg[k] and seg[k] >= 0   (Python chained compare)
    keep_noise(q,k)  : noise[k] < 0 or noise[q] == noise[k]
    same_sample(q,k) : sample[q] == sample[k]
W is the per-layer sliding window; a global layer uses W = infinity (here any
W >= the sequence length, e.g. 0x7fffffff, behaves identically).

Pinned by: tests/test_oracle_mask.py (against a span-level reading of the mode
table in the same section, by brute force over random tiny layouts; sample
isolation; closed-form legal-key counts per query).
"""
from __future__ import annotations

import numpy as np


def legal(q_tracks, k_tracks, window: int) -> np.ndarray:
    """Boolean matrix [nq, nk]: may query i attend key j.

    q_tracks, k_tracks: tuples (sample, seg, noise, pos) of int arrays.
    Evaluated with torch's CPU integer ops (threaded) on int32 copies of the
    tracks; the result is a numpy bool array.
    """
    import torch
    qs, qg, qn, qp = (torch.from_numpy(np.ascontiguousarray(a, np.int32))[:, None] for a in q_tracks)
    ks, kg, kn, kp = (torch.from_numpy(np.ascontiguousarray(a, np.int32))[None, :] for a in k_tracks)
    diff = qp - kp          # positions are non-negative int32: no overflow
    causal = (diff >= 0) & (diff < min(int(window), 0x7FFFFFFF))
    same_span = (qg == kg) & (kg >= 0)
    keep_noise = (kn < 0) | (qn == kn)
    same_sample = qs == ks
    return ((causal | same_span) & keep_noise & same_sample).numpy()


def take(tracks, idx):
    """Tracks restricted to token indices `idx` (any order)."""
    return tuple(np.asarray(a)[idx] for a in tracks)
