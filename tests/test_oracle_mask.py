"""Pins of the mask predicate (oracle/mask.py).

The predicate is checked against a span-level reading of the mode table in
MARBLE section 01 (the table of the five modes and the prose around it),
written independently of the four-track formula: a pair is legal when
  * both tokens are in one sample (no sample attends another),
  * the key is not in a generated (noise) span, unless it is the query's own
    noise span (a noise span is "not seen later"),
  * and either they are in the same span and the span's mode allows it
    (bidirectional modes: always; causal / window: key not after the query and
    within the window), or they are spans of one group (all group spans see
    each other), or the key's span is earlier in the sample and the key lies
    within the layer window of the query ("later spans may attend to earlier
    ones"; window layers only within W).
"""
import numpy as np
import pytest

from workloads import random_small, sliding_window, packed_text, WINDOW_INF
from oracle.mask import legal


def semantic_legal(spans, n, window):
    span_of = np.empty(n, np.int64)
    for i, (a, b, mode, smp) in enumerate(spans):
        span_of[a:b] = i
    # group membership: group spans of one sample share their group
    group = {}
    for i, (a, b, mode, smp) in enumerate(spans):
        if mode == "group":
            group[i] = ("g", smp)
    out = np.zeros((n, n), bool)
    for q in range(n):
        sq = span_of[q]
        aq, bq, mq, smpq = spans[sq]
        for k in range(n):
            sk = span_of[k]
            ak, bk, mk, smpk = spans[sk]
            if smpq != smpk:
                continue
            if mk == "noise" and sk != sq:
                continue
            if sk == sq:
                if mq in ("full", "noise", "group"):
                    out[q, k] = True
                else:
                    out[q, k] = 0 <= q - k < window
                continue
            if sq in group and sk in group and group[sq] == group[sk]:
                out[q, k] = True
                continue
            if ak < aq:
                out[q, k] = 0 <= q - k < window
    return out


@pytest.mark.parametrize("seed", range(40))
def test_predicate_matches_mode_table(seed):
    rng = np.random.default_rng(seed)
    lay = random_small(rng, int(rng.integers(8, 48)))
    want = semantic_legal(lay.spans, lay.n, lay.window)
    got = legal(lay.tracks(), lay.tracks(), lay.window)
    assert np.array_equal(got, want)


def test_no_cross_sample_pairs():
    lay = packed_text(n=4096, seed=5, ranks=4)
    m = legal(lay.tracks(), lay.tracks(), lay.window)
    smp = lay.sample
    assert not (m & (smp[:, None] != smp[None, :])).any()
    # every token sees itself
    assert m.diagonal().all()


def test_causal_counts_closed_form():
    """Causal text: query at offset t of its document sees t + 1 keys."""
    lay = packed_text(n=4096, seed=6, ranks=4)
    m = legal(lay.tracks(), lay.tracks(), lay.window)
    off = np.zeros(lay.n, np.int64)
    for a, b, mode, smp in lay.spans:
        off[a:b] = np.arange(b - a)
    assert np.array_equal(m.sum(1), off + 1)


def test_window_counts_closed_form():
    """Clip-bidirectional + sliding window W: offset t sees the whole clip plus
    max(0, W - 1 - t) keys of the previous clip of its document."""
    clip, w = 64, 16
    lay = sliding_window(n=512, clip=clip, clips_per_doc=4, window=w, ranks=8)
    m = legal(lay.tracks(), lay.tracks(), lay.window)
    t = np.arange(lay.n) % clip
    c = np.arange(lay.n) // clip
    prev = np.where(c % 4 > 0, np.maximum(0, w - 1 - t), 0)
    assert np.array_equal(m.sum(1), clip + prev)
