"""Ring attention for one rank, simulated step by step with a carried state.

Follows the ring-attention explainer ("Sequence Partitioning", "Execution
Algorithm", "The Online Softmax Formulation") and the NumPy ring page ("The
whole algorithm, simulated"): the rank keeps its query shard, at step s it
holds the key/value shard of rank j = (r - s) mod P, and it folds that shard
into a running state (m, l, O):
    m'  = max(m, rowmax of s over shard j's legal keys)
    c   = exp(m - m')            (c := 1 when m' = -inf: nothing seen yet)
    l   = c * l + sum exp(s - m')
    O   = c * O + sum exp(s - m') v
    m   = m'
and only after the last step normalizes: O / l and LSE = m + ln l.  The state
is kept unnormalized, as MARBLE's online kernel keeps it (MARBLE, section 03
"Exact ring attention accumulation"), and no epsilon is added to l.

The step order is the ring's; masking is per token pair with the same predicate
as the single-pass definition, so the result equals single-pass attention up to
rounding (the merge is associative).

Pinned by: tests/test_oracle_ring.py (the NumPy page's printed toy result:
allclose at 1e-5 and 256 B / 1024 B of key/value bytes; fp64 ring equals the
fp64 direct definition to 1e-12 on masked layouts).
"""
from __future__ import annotations

import numpy as np

from .attention import as_f64, gather, kv_head
from .mask import legal, take


class RingState:
    """Unnormalized running state of one rank: m, l [Hq, S]; O [S, Hq, d]."""

    def __init__(self, s: int, hq: int, d: int, dtype=np.float64):
        self.dtype = dtype
        self.m = np.full((hq, s), -np.inf, dtype)
        self.l = np.zeros((hq, s), dtype)
        self.o = np.zeros((s, hq, d), dtype)

    def fold(self, q, k, v, allowed, scale):
        """Fold one key/value shard into the state (one ring step)."""
        dt = self.dtype
        hq, hkv = q.shape[1], k.shape[1]
        for h in range(hq):
            g = kv_head(h, hq, hkv)
            s = (q[:, h, :] @ k[:, g, :].T) * dt(scale)
            s = np.where(allowed, s, dt(-np.inf))
            row_max = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf, dt)
            m_new = np.maximum(self.m[h], row_max)
            seen = np.isfinite(m_new)
            base = np.where(seen, m_new, dt(0))
            c = np.where(seen, np.exp(self.m[h] - base), dt(1))
            p = np.exp(s - base[:, None])
            self.l[h] = c * self.l[h] + p.sum(axis=1)
            self.o[:, h, :] = c[:, None] * self.o[:, h, :] + p @ v[:, g, :]
            self.m[h] = m_new

    def finish(self):
        """O = O / l, LSE = m + ln l (O = 0, LSE = -inf where l = 0)."""
        l = self.l
        with np.errstate(invalid="ignore", divide="ignore"):
            o = np.where((l.T > 0)[:, :, None], self.o / l.T[:, :, None], 0)
            lse = np.where(l > 0, self.m + np.log(l), -np.inf)
        return o.astype(self.dtype), lse.astype(self.dtype)


def ring_share(tracks, window: int, q, k, v, perm, ranks: int, r: int, scale: float,
               dtype=np.float64, steps=None):
    """One rank's share, P steps: queries perm[rS:(r+1)S], keys of shard (r-s) mod P.

    q, k, v are full arrays in the ORIGINAL order; `perm[new] = original`.
    Returns (O [S,Hq,d], LSE [Hq,S]) in the rank's (new) order.
    """
    perm = np.asarray(perm, np.int64)
    n = len(perm)
    s_tok = n // ranks
    rows = perm[r * s_tok:(r + 1) * s_tok]
    conv = (lambda x: as_f64(x).astype(dtype))
    qr = conv(gather(q, rows))
    st = RingState(len(rows), q.shape[1], v.shape[2], dtype)
    qt = take(tracks, rows)
    for s in (range(ranks) if steps is None else steps):
        j = (r - s) % ranks
        keys = perm[j * s_tok:(j + 1) * s_tok]
        allowed = legal(qt, take(tracks, keys), window)
        st.fold(qr, conv(gather(k, keys)), conv(gather(v, keys)), allowed, scale)
    return st.finish()


def toy_ring_fp32(q, k, v, ranks: int):
    """The unmasked fp32 ring of the NumPy page on contiguous shards.

    Returns (ring output [N, d], largest key/value shard bytes, whole K+V bytes).
    """
    n, d = q.shape
    s_tok = n // ranks
    scale = np.float32(1.0 / np.sqrt(d))
    out = []
    peak = 0
    for r in range(ranks):
        st = RingState(s_tok, 1, d, np.float32)
        qr = q[r * s_tok:(r + 1) * s_tok, None, :].astype(np.float32)
        for s in range(ranks):
            j = (r - s) % ranks
            kb = k[j * s_tok:(j + 1) * s_tok].astype(np.float32)
            vb = v[j * s_tok:(j + 1) * s_tok].astype(np.float32)
            peak = max(peak, kb.nbytes + vb.nbytes)
            st.fold(qr, kb[:, None, :], vb[:, None, :],
                    np.ones((s_tok, s_tok), bool), scale)
        o, _ = st.finish()
        out.append(o[:, 0, :])
    return np.concatenate(out), peak, k.astype(np.float32).nbytes + v.astype(np.float32).nbytes
