"""Pins of the fp64 gradients (oracle/backward.py): central finite differences."""
import numpy as np
import pytest

from workloads import random_small
from oracle import attention, backward


def _loss(tr, w, q, k, v, do, rows, scale):
    o, _ = attention.forward_rows(tr, w, q, k, v, rows, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("seed", range(3))
def test_finite_differences(seed):
    rng = np.random.default_rng(seed)
    lay = random_small(rng, 24)
    tr = lay.tracks()
    n, hq, hkv, d = lay.n, 4, 2, 4
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((n, hkv, d))
    v = rng.standard_normal((n, hkv, d))
    do = rng.standard_normal((n, hq, d))
    rows = np.sort(rng.choice(n, size=n // 2, replace=False))
    scale = 0.37
    # chunks of 5 rows: every chunk's key restriction is exercised
    g = backward.backward_rows(tr, lay.window, q, k, v, do, rows, scale, chunk=5)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for a, b, dkb, dvb in g["dkv"]:
        dk[a:b] += dkb
        dv[a:b] += dvb
    dq = np.zeros_like(q)
    dq[rows] = g["dq"]
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in x.shape)
            old = x[idx]
            x[idx] = old + h
            lp = _loss(tr, lay.window, q, k, v, do[rows], rows, scale)
            x[idx] = old - h
            lm = _loss(tr, lay.window, q, k, v, do[rows], rows, scale)
            x[idx] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_delta_and_unread_keys():
    rng = np.random.default_rng(8)
    lay = random_small(rng, 30)
    tr = lay.tracks()
    n = lay.n
    q = rng.standard_normal((n, 2, 4))
    k = rng.standard_normal((n, 1, 4))
    v = rng.standard_normal((n, 1, 4))
    do = rng.standard_normal((n, 2, 4))
    rows = np.arange(0, n, 2)
    g = backward.backward_rows(tr, lay.window, q, k, v, do, rows, 0.5, chunk=4)
    np.testing.assert_allclose(g["delta"], (g["o"] * do[rows]).sum(-1).T, atol=1e-13)
    from oracle.mask import legal, take
    m = legal(take(tr, rows), tr, lay.window)
    read = m.any(0)
    dk = np.zeros_like(k)
    for a, b, dkb, dvb in g["dkv"]:
        dk[a:b] += dkb
    assert np.all(dk[~read] == 0)


@pytest.mark.parametrize("seed", range(3))
def test_key_sum_identities(seed):
    """Summed over every key: dV gives the summed dO of the rows that read a
    key (each row of P sums to 1), and dK gives zero (sum_j dS_ij =
    dO_i . O_i - D_i = 0), per key/value head over its group of query heads."""
    rng = np.random.default_rng(40 + seed)
    lay = random_small(rng, 40)
    tr = lay.tracks()
    n, hq, hkv, d = lay.n, 6, 2, 5
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((n, hkv, d))
    v = rng.standard_normal((n, hkv, d))
    do = rng.standard_normal((n, hq, d))
    rows = np.sort(rng.choice(n, size=2 * n // 3, replace=False))
    g = backward.backward_rows(tr, lay.window, q, k, v, do, rows, 0.61, chunk=7)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for a, b, dkb, dvb in g["dkv"]:
        dk[a:b] += dkb
        dv[a:b] += dvb
    from oracle.mask import legal, take
    live = legal(take(tr, rows), tr, lay.window).any(1)     # rows with a legal key
    do_live = do[rows][live]                                 # [rows, hq, d]
    want = do_live.sum(0).reshape(hkv, hq // hkv, d).sum(1)
    np.testing.assert_allclose(dv.sum(0), want, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk.sum(0), 0.0, rtol=0, atol=1e-11)
    assert np.abs(dk).max() > 1e-2                           # the identity is not vacuous


def test_forward_terms_match_the_forward_oracle():
    """O and LSE that the backward evaluates (chunked, keys restricted) equal
    the forward oracle's (numpy, all keys of each sample) to fp64 rounding."""
    rng = np.random.default_rng(12)
    lay = random_small(rng, 200, max_span=60)
    tr = lay.tracks()
    n = lay.n
    q = rng.standard_normal((n, 4, 8))
    k = rng.standard_normal((n, 2, 8))
    v = rng.standard_normal((n, 2, 8))
    do = rng.standard_normal((n, 4, 8))
    rows = np.sort(rng.choice(n, size=150, replace=False))
    g = backward.backward_rows(tr, lay.window, q, k, v, do, rows, 0.3, chunk=9)
    o, lse = attention.forward_rows(tr, lay.window, q, k, v, rows, 0.3)
    np.testing.assert_allclose(g["o"], o, rtol=0, atol=1e-12)
    fin = np.isfinite(lse)
    assert np.array_equal(np.isfinite(g["lse"]), fin)
    np.testing.assert_allclose(g["lse"][fin], lse[fin], rtol=0, atol=1e-12)
