"""Pins of the oracle's ring iteration (oracle/ring.py)."""
import numpy as np
import pytest

from workloads import toy_qkv, random_small, packed_text
from oracle import ring, attention, planner
from goldens import read


def _reference_unmasked(q, k, v):
    # Plain softmax attention written with scipy's softmax (an independent routine).
    from scipy.special import softmax
    s = (q.astype(np.float64) @ k.astype(np.float64).T) / np.sqrt(q.shape[1])
    return softmax(s, axis=-1) @ v.astype(np.float64)


def test_toy_matches_printed_output():
    """NumPy ring page, printed output: allclose(atol=1e-5) True, max diff ~1.79e-7,
    256 B largest K/V shard, 1024 B whole K/V."""
    g = read("numpy_ring_toy.txt")
    q, k, v = toy_qkv()
    out, peak, whole = ring.toy_ring_fp32(q, k, v, int(g["devices"]))
    ref = _reference_unmasked(q, k, v)
    diff = float(np.abs(out - ref).max())
    assert (diff <= 1e-5) == (g["allclose_atol_1e-5"] == "True")
    # same order of magnitude as the printed fp32 difference (BLAS order differs)
    assert diff < 10 * float(g["max_difference"])
    assert peak == int(g["largest_kv_in_flight_bytes"])
    assert whole == int(g["whole_sequence_kv_bytes"])
    assert out.shape[0] // int(g["devices"]) == int(g["tokens_per_device"])


def test_toy_fp64_ring_equals_direct():
    q, k, v = toy_qkv()
    lay_tracks = (np.zeros(16, np.int32), np.zeros(16, np.int32), -np.ones(16, np.int32),
                  np.arange(16, dtype=np.int32))
    perm = np.arange(16)
    scale = 1 / np.sqrt(8)
    for r in range(4):
        o, lse = ring.ring_share(lay_tracks, 0x7FFFFFFF, q[:, None, :], k[:, None, :],
                                 v[:, None, :], perm, 4, r, scale)
        od, ld = attention.forward_rows(lay_tracks, 0x7FFFFFFF, q[:, None, :], k[:, None, :],
                                        v[:, None, :], perm[4 * r:4 * r + 4], scale)
        np.testing.assert_allclose(o, od, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse, ld, atol=1e-12, rtol=0)


@pytest.mark.parametrize("seed", range(6))
def test_masked_ring_fp64_equals_direct(seed):
    """Associativity of the merge (ring-attention explainer, Online Softmax):
    the fp64 ring over masked shards equals the direct definition."""
    rng = np.random.default_rng(100 + seed)
    ranks = [1, 2, 3, 4][seed % 4]
    n = 8 * ranks * 4
    lay = random_small(rng, n)
    tr = lay.tracks()
    hq, hkv, d = 4, 2, 8
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((n, hkv, d))
    v = rng.standard_normal((n, hkv, d))
    order = "ptrr" if seed % 2 else "contiguous"
    p = planner.build(tr, lay.window, ranks, 8, order)
    for r in range(ranks):
        o, lse = ring.ring_share(tr, lay.window, q, k, v, p.perm, ranks, r, 0.3)
        rows = p.perm[r * (n // ranks):(r + 1) * (n // ranks)]
        od, ld = attention.forward_rows(tr, lay.window, q, k, v, rows, 0.3)
        np.testing.assert_allclose(o, od, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse, ld, atol=1e-12, rtol=0)


def test_packed_text_ring_equals_direct_subset():
    """fp64 ring == direct on a shortened packed-text layout (same recipe)."""
    lay = packed_text(n=4096, seed=2, ranks=4)
    tr = lay.tracks()
    rng = np.random.default_rng(7)
    q = rng.standard_normal((lay.n, 2, 16))
    k = rng.standard_normal((lay.n, 1, 16))
    v = rng.standard_normal((lay.n, 1, 16))
    p = planner.build(tr, lay.window, 4, 128, "ptrr")
    r = p.busiest_rank()
    o, lse = ring.ring_share(tr, lay.window, q, k, v, p.perm, 4, r, 0.25)
    rows = p.perm[r * 1024:(r + 1) * 1024]
    od, ld = attention.forward_rows(tr, lay.window, q, k, v, rows, 0.25)
    np.testing.assert_allclose(o, od, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, ld, atol=1e-12, rtol=0)


def test_fp32_carry_beats_bf16_merge():
    """MARBLE section 03: rounding normalized partial outputs to bf16 at every
    step adds error that the fp32 carry does not have."""
    import torch
    lay = packed_text(n=2048, seed=3, ranks=8)
    tr = lay.tracks()
    rng = np.random.default_rng(11)
    q = rng.standard_normal((lay.n, 1, 32)).astype(np.float32)
    k = rng.standard_normal((lay.n, 1, 32)).astype(np.float32)
    v = rng.standard_normal((lay.n, 1, 32)).astype(np.float32)
    p = planner.build(tr, lay.window, 8, 128, "ptrr")
    r = p.busiest_rank()
    s_tok = lay.n // 8
    rows = p.perm[r * s_tok:(r + 1) * s_tok]
    ref, _ = attention.forward_rows(tr, lay.window, q, k, v, rows, 1 / np.sqrt(32))
    o32, _ = ring.ring_share(tr, lay.window, q, k, v, p.perm, 8, r, 1 / np.sqrt(32),
                             dtype=np.float32)
    # per-step normalized outputs rounded to bf16 and merged with an LSE rescale
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()
    o_m = None
    lse_m = None
    from oracle.mask import legal, take
    for s in range(8):
        j = (r - s) % 8
        keys = p.perm[j * s_tok:(j + 1) * s_tok]
        st = ring.RingState(s_tok, 1, 32, np.float64)
        st.fold(q[rows].astype(np.float64), k[keys].astype(np.float64),
                v[keys].astype(np.float64), legal(take(tr, rows), take(tr, keys), lay.window),
                1 / np.sqrt(32))
        o_s, lse_s = st.finish()
        o_s = bf(o_s)
        if o_m is None:
            o_m, lse_m = o_s, lse_s
            continue
        new = np.logaddexp(lse_m, lse_s)
        with np.errstate(invalid="ignore"):
            w1 = np.where(np.isfinite(lse_m), np.exp(lse_m - new), 0.0)
            w2 = np.where(np.isfinite(lse_s), np.exp(lse_s - new), 0.0)
        o_m = bf(w1.T[:, :, None] * o_m + w2.T[:, :, None] * o_s)
        lse_m = new
    err_carry = np.abs(bf(o32) - ref).mean()
    err_merge = np.abs(o_m - ref).mean()
    assert err_merge > err_carry
