"""Pins of the fp64 attention definition (oracle/attention.py)."""
import numpy as np
import pytest
import torch

from workloads import random_small, packed_multimodal, packed_text
from oracle import attention, planner
from oracle.mask import legal


def _rand_layout(seed, n=40):
    rng = np.random.default_rng(seed)
    return rng, random_small(rng, n)


@pytest.mark.parametrize("seed", range(5))
def test_rows_sum_to_one_and_zero_outside_mask(seed):
    """With V = identity over keys, O's rows are the softmax rows: they sum to 1
    and vanish on illegal pairs (in particular across samples)."""
    rng, lay = _rand_layout(seed)
    n = lay.n
    q = rng.standard_normal((n, 1, 8))
    k = rng.standard_normal((n, 1, 8))
    v = np.eye(n)[:, None, :]
    o, _ = attention.forward_rows(lay.tracks(), lay.window, q, k, v, np.arange(n), 0.4)
    p = o[:, 0, :]
    np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-12)
    m = legal(lay.tracks(), lay.tracks(), lay.window)
    assert np.all(p[~m] == 0.0)
    assert np.all(p[m] > 0.0)


@pytest.mark.parametrize("seed", range(5))
def test_zero_query_gives_log_count(seed):
    """Q = 0: every legal score is 0, so l_i = n_i and LSE_i = ln n_i, O_i = mean of legal V."""
    rng, lay = _rand_layout(seed)
    n = lay.n
    q = np.zeros((n, 2, 8))
    k = rng.standard_normal((n, 1, 8))
    v = rng.standard_normal((n, 1, 8))
    o, lse = attention.forward_rows(lay.tracks(), lay.window, q, k, v, np.arange(n), 0.4)
    m = legal(lay.tracks(), lay.tracks(), lay.window)
    cnt = m.sum(1)
    np.testing.assert_allclose(lse[0], np.log(cnt), atol=1e-13)
    mean_v = (m.astype(np.float64) @ v[:, 0, :]) / cnt[:, None]
    np.testing.assert_allclose(o[:, 1, :], mean_v, atol=1e-13)


def test_unit_values_give_unit_output():
    rng, lay = _rand_layout(9)
    n = lay.n
    q = rng.standard_normal((n, 2, 8))
    k = rng.standard_normal((n, 2, 8))
    o, _ = attention.forward_rows(lay.tracks(), lay.window, q, k, np.ones((n, 2, 8)),
                                  np.arange(n), 0.4)
    np.testing.assert_allclose(o, 1.0, atol=1e-13)


def test_dense_case_matches_torch_sdpa():
    """An unmasked single sample reduces to plain scaled-dot-product attention
    (torch's CPU routine, fp64)."""
    rng = np.random.default_rng(3)
    n, hq, hkv, d = 50, 4, 2, 16
    tr = (np.zeros(n, np.int32), np.zeros(n, np.int32), -np.ones(n, np.int32),
          np.arange(n, dtype=np.int32))
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((n, hkv, d))
    v = rng.standard_normal((n, hkv, d))
    o, _ = attention.forward_rows(tr, 0x7FFFFFFF, q, k, v, np.arange(n), 1 / np.sqrt(d))
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_causal_case_matches_torch_sdpa():
    """One causal document reduces to SDPA with is_causal=True."""
    rng = np.random.default_rng(4)
    n, d = 64, 16
    tr = (np.zeros(n, np.int32), -np.ones(n, np.int32), -np.ones(n, np.int32),
          np.arange(n, dtype=np.int32))
    q = rng.standard_normal((n, 1, d))
    k = rng.standard_normal((n, 1, d))
    v = rng.standard_normal((n, 1, d))
    o, _ = attention.forward_rows(tr, 0x7FFFFFFF, q, k, v, np.arange(n), 1 / np.sqrt(d))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(k).permute(1, 0, 2),
        torch.from_numpy(v).permute(1, 0, 2), is_causal=True).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_layout_invariance():
    """MARBLE section 04 'Layout transforms': permuting tokens (with their
    tracks) leaves every query's result unchanged."""
    lay = packed_multimodal(n=4096, seed=3, ranks=4)
    tr = lay.tracks()
    rng = np.random.default_rng(5)
    q = rng.standard_normal((lay.n, 2, 8))
    k = rng.standard_normal((lay.n, 2, 8))
    v = rng.standard_normal((lay.n, 2, 8))
    p = planner.build(tr, lay.window, 4, 128, "ptrr")
    rows = np.arange(0, lay.n, 7)
    o1, l1 = attention.forward_rows(tr, lay.window, q, k, v, rows, 0.3)
    # evaluate in the permuted order: tracks and tensors permuted together
    inv = np.argsort(p.perm)
    trp = tuple(a[p.perm] for a in tr)
    # the permuted order breaks sample contiguity, so evaluate densely
    allowed = legal(tuple(a[inv[rows]] for a in trp), trp, lay.window)
    o2, l2 = attention.attention_fp64(q[p.perm][inv[rows]], k[p.perm], v[p.perm], allowed, 0.3)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


def test_legal_counts_closed_forms():
    """legal_counts (the checker of the GPU zero-query test) against counts
    that follow from the layouts' structure alone: a causal text document
    gives query i of a document starting at a exactly i - a + 1 keys; a clip
    under the sliding window sees its whole clip, plus the last W - 1 - t keys
    of the previous clip of its document at offset t < W - 1 in the clip."""
    from workloads import sliding_window
    lay = packed_text()
    rng = np.random.default_rng(4)
    rows = np.sort(rng.choice(lay.n, 300, replace=False))
    start = {}
    for a, b, mode, sid in lay.spans:
        assert mode == "causal"
        start[sid] = a
    want = rows - np.array([start[int(lay.sample[t])] for t in rows]) + 1
    assert np.array_equal(attention.legal_counts(lay.tracks(), lay.window, rows), want)
    clip, w = 2048, 512
    lay = sliding_window(n=16384, clip=clip, window=w)
    rows = np.concatenate([np.arange(0, 2 * clip, 97), np.arange(clip, clip + w + 3),
                           rng.choice(lay.n, 200, replace=False)])
    c, t = rows // clip, rows % clip
    prev_same_doc = (c % 4) != 0
    want = clip + np.where(prev_same_doc, np.maximum(0, w - 1 - t), 0)
    assert np.array_equal(attention.legal_counts(lay.tracks(), lay.window, rows), want)
