"""GPU parity of the forward ring steps against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import block_sparse_masked_metadata_amd as bsm
from workloads import (ring_toy, toy_qkv, random_small, packed_text, packed_multimodal,
                       sliding_window, long_mixed)
from oracle import attention as oatt
from oracle.mask import legal, take
from gpu_common import Case, O_TOL, LSE_TOL, check_rows, max_err, needs_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not needs_gpu, reason="needs a GPU")]


def _check_rows(case, o, lse, sel=None, tol_o=O_TOL, tol_lse=LSE_TOL):
    return check_rows(case, o, lse, sel, tol_o, tol_lse)


def test_ring_toy():
    """The NumPy page's 16-token, 4-rank toy: inputs rounded to bf16 and the
    head dim zero-padded 8 -> 128 (exact), scale 1/sqrt(8), every rank."""
    lay = ring_toy()
    q8, k8, v8 = toy_qkv()
    pad = lambda x: torch.nn.functional.pad(torch.from_numpy(x), (0, 120)).to(torch.bfloat16)[:, None, :]
    t = tuple(pad(x).cuda() for x in (q8, k8, v8))
    for r in range(4):
        case = Case(lay, rank=r, tensors=t)
        o, lse, _ = case.ring()
        torch.cuda.synchronize()
        _check_rows(case, o, lse)
        assert torch.all(o[:, :, 8:] == 0)


@pytest.mark.parametrize("seed", range(6))
def test_random_layouts_all_modes(seed):
    rng = np.random.default_rng(900 + seed)
    ranks = [1, 2, 4, 3, 8, 2][seed]
    order = ["ptrr", "contiguous"][seed % 2]
    n = 128 * ranks * [2, 3, 1, 2, 1, 4][seed]
    lay = random_small(rng, n, max_span=300)
    lay.ranks, lay.order, lay.seed = ranks, order, 40 + seed
    lay.hq, lay.hkv = [(4, 2), (2, 2), (8, 1), (4, 4), (6, 3), (2, 1)][seed]
    lay.d = 128
    for r in range(ranks):
        case = Case(lay, rank=r)
        o, lse, _ = case.ring()
        torch.cuda.synchronize()
        _check_rows(case, o, lse)


def test_packed_text_full_share():
    case = Case(packed_text())
    o, lse, _ = case.ring()
    torch.cuda.synchronize()
    _check_rows(case, o, lse)


def test_packed_multimodal_full_share():
    case = Case(packed_multimodal())
    o, lse, _ = case.ring()
    torch.cuda.synchronize()
    _check_rows(case, o, lse)


def test_sliding_window_full_size_sampled():
    case = Case(sliding_window())
    o, lse, _ = case.ring()
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    sel = np.concatenate([np.arange(0, 4200, 97), rng.choice(case.S, 200, replace=False)])
    _check_rows(case, o, lse, np.unique(sel))


def test_long_mixed_full_size_sampled():
    case = Case(long_mixed())
    o, lse, _ = case.ring()
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    _check_rows(case, o, lse, np.sort(rng.choice(case.S, 256, replace=False)))


def test_ring_equals_single_bitwise():
    """The carried fp32 state makes the ring equal the single pass exactly
    (MARBLE section 03: ring output equals a single GPU's)."""
    for lay in (packed_multimodal(), packed_text()):
        case = Case(lay)
        _, _, st_ring = case.ring(keep_state=True)
        st_single = case.single(keep_state=True)
        o1, l1, _ = case.ring()
        o2, l2 = case.single()
        torch.cuda.synchronize()
        for a, b in zip(st_ring, st_single):
            assert torch.equal(a, b)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_state_host_round_trip_resume():
    """Stop after 4 steps, move the state to the host, free it, upload it into
    fresh buffers and finish: bitwise equal to the uninterrupted ring.  (Tiles
    whose last step is early write O/LSE during the first half, so both halves
    share the output buffers.)"""
    case = Case(packed_multimodal())
    o_ref, l_ref, _ = case.ring()
    o = torch.full_like(o_ref, float("nan"))
    l = torch.full_like(l_ref, float("nan"))
    _, _, st = case.ring(steps=range(4), out=(o, l))
    host = [t.cpu() for t in st]
    del st
    torch.cuda.empty_cache()
    st2 = tuple(t.cuda() for t in host)
    case.ring(steps=range(4, 8), state=st2, out=(o, l))
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


def test_unit_values_and_zero_queries():
    """V = 1 gives O = 1; Q = 0 gives LSE = ln(#legal keys) per row, where the
    count is the mask's, and O = mean of the legal values."""
    lay = packed_multimodal()
    base = Case(lay)
    q0 = torch.zeros_like(base.full[0])
    ones = torch.ones_like(base.full[2])
    case = Case(lay, tensors=(base.full[0], base.full[1], ones))
    o, lse, _ = case.ring()
    torch.cuda.synchronize()
    assert float((o.float() - 1).abs().max()) <= 1e-2
    case = Case(lay, tensors=(q0, base.full[1], base.full[2]))
    o, lse, _ = case.ring()
    torch.cuda.synchronize()
    sel = np.arange(0, case.S, 37)
    cnt = oatt.legal_counts(lay.tracks(), lay.window, case.rows[sel])
    lg = lse[:, torch.from_numpy(sel).cuda()].cpu().numpy()
    np.testing.assert_allclose(lg, np.broadcast_to(np.log(cnt), lg.shape), rtol=2e-6)
    _check_rows(case, o, lse, sel)


def test_sample_isolation_exact():
    """V = 1 on one sample and 0 elsewhere: rows of other samples get exactly 0;
    perturbing other samples' K/V leaves the sample's rows bitwise unchanged."""
    lay = packed_text()
    base = Case(lay)
    smp = torch.from_numpy(lay.sample.astype(np.int64)).cuda()
    target = int(lay.sample[base.rows[0]])
    vsel = torch.where((smp == target)[:, None, None], 1.0, 0.0).to(torch.bfloat16)
    vsel = vsel.expand_as(base.full[2]).contiguous()
    case = Case(lay, tensors=(base.full[0], base.full[1], vsel))
    o, _, _ = case.ring()
    torch.cuda.synchronize()
    mine = torch.from_numpy(lay.sample[case.rows] == target).cuda()
    assert torch.all(o[~mine] == 0)
    o_ref, l_ref, _ = base.ring()
    k2 = base.full[1].clone()
    v2 = base.full[2].clone()
    other = (smp != target)
    k2[other] = k2[other] * 3 + 1
    v2[other] = -v2[other]
    pert = Case(lay, tensors=(base.full[0], k2, v2))
    o2, l2, _ = pert.ring()
    torch.cuda.synchronize()
    assert torch.equal(o2[mine], o_ref[mine]) and torch.equal(l2[:, mine], l_ref[:, mine])


def test_layout_invariance_ptrr_vs_contiguous():
    """Same keys per query in either token order: outputs agree per original token."""
    lay = packed_text()
    a = Case(lay)
    lay_c = packed_text()
    lay_c.order = "contiguous"
    outs = {}
    for c in [a] + [Case(lay_c, rank=r, tensors=a.full) for r in range(lay.ranks)]:
        o, lse, _ = c.ring()
        torch.cuda.synchronize()
        for i, t in enumerate(c.rows[:: 61]):
            outs.setdefault(int(t), []).append(o[i * 61].float().cpu())
    for t, vals in outs.items():
        for v in vals[1:]:
            assert float((v - vals[0]).abs().max()) <= 1e-2


def test_fwd_errors_before_launch():
    case = Case(packed_text())
    C = bsm._capi
    hd = bsm.heads(32, 8, 64)
    with pytest.raises(bsm.BsmError) as e:
        C.bsm_fwd_single(case.dp.handle, hd, case.q.data_ptr(), case.k_all.data_ptr(),
                         case.v_all.data_ptr(), None, None, None, case.q.data_ptr(),
                         case.q.data_ptr(), 0, None)
    assert e.value.code == C.BSM_E_UNSUPPORTED
    acc, m, l = bsm.new_state(case.S, case.hq, 128)
    o, lse = torch.empty_like(case.q), torch.empty_like(m)
    ptrs = [t.data_ptr() for t in (case.q, case.k_shards[0], case.v_shards[0], acc, m, l, o, lse)]
    with pytest.raises(bsm.BsmError) as e:
        C.bsm_fwd_step(case.dp.handle, 99, case.heads, *ptrs, 0, None)
    assert e.value.code == C.BSM_E_INVALID
    # 4096 shard rows x 4096 heads x 256 B = 4 GiB per bf16 tensor: refused before
    # any launch.  The buffers are real and as large as such a call would address,
    # so nothing would fault even if the refusal went missing.
    big = bsm.heads(4096, 4096)
    bf = torch.empty(case.S * 4096 * 128, dtype=torch.bfloat16, device="cuda")
    f32 = torch.empty(case.S * 4096 * 128, dtype=torch.float32, device="cuda")
    rowf = torch.empty(4096 * case.S, dtype=torch.float32, device="cuda")
    B, F, W = bf.data_ptr(), f32.data_ptr(), rowf.data_ptr()
    for fn in (lambda: C.bsm_fwd_step(case.dp.handle, 0, big, B, B, B, F, W, W, B, W, 0, None),
               lambda: C.bsm_bwd_step(case.dp.handle, 0, big, B, B, B, B, W, W, F, F, F, None)):
        with pytest.raises(bsm.BsmError) as e:
            fn()
        assert e.value.code == C.BSM_E_UNSUPPORTED
        assert "4 GiB" in str(e.value)
    del bf, f32, rowf
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_state_unpack_channel_order():
    """V[k, kvh, c] = c makes every reached row's O_acc / l a weighted mean
    of c with weights bf16(p) / sum p, i.e. c within 2^-9 relative (P is
    rounded to bf16 for the product, l sums the fp32 p).  Channels differ by
    at least 1, so this pins the channel order of the tile-blocked state read
    back through bsm_state_unpack (rows and heads are pinned by the oracle
    comparisons above)."""
    lay = packed_text()
    base = Case(lay)
    v = torch.arange(128, dtype=torch.float32, device="cuda").to(torch.bfloat16)
    v = v.expand_as(base.full[2]).contiguous()
    case = Case(lay, tensors=(base.full[0], base.full[1], v))
    _, _, (acc, m, l) = case.ring(keep_state=True)
    rows = bsm.state_rows(case.heads, acc, case.S)
    torch.cuda.synchronize()
    lt = l.T[:, :, None]
    assert bool((lt > 0).all())
    want = torch.arange(128, dtype=torch.float32, device="cuda").expand_as(rows)
    assert bool((((rows / lt) - want).abs() <= want * 2.0 ** -8 + 1e-3).all())


def test_mfma_probe_reports_a_plausible_rate_and_clock():
    """The measurement probe (libbsm_probe.so) runs and reads back sane numbers."""
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    pr = bench.mfma_probe(torch)
    assert pr is not None, "libbsm_probe.so is not built"
    assert 100.0 < pr["tflops"] < 3000.0
    assert 0.5 < pr["clock_ghz"] < 3.0


def test_key_rows_past_2gib():
    """Key and value buffers of 2.5 GiB (1,310,720 tokens x 8 kv heads x 256 B):
    the full sub-tiles of the last query tiles read rows more than 2 GiB into
    them.  One sample under a 256-token sliding window, single pass; sampled rows
    of the last tiles against the oracle on the token slice that holds every key
    they read (the mask depends on positions and samples only)."""
    from workloads.layouts import Layout
    n, h, w = 1310720, 8, 256
    neg = np.full(n, -1, np.int32)
    lay = Layout("window_2p5gib", sample=np.zeros(n, np.int32), seg=neg, noise=neg.copy(),
                 pos=np.arange(n, dtype=np.int32), window=w, ranks=1, order="contiguous",
                 hq=h, hkv=h, seed=21)
    case = Case(lay)
    assert case.k_all.numel() * case.k_all.element_size() > 2 ** 31 + 2 ** 28
    o, lse = case.single()
    torch.cuda.synchronize()
    sel = np.arange(n - 512, n, 7)
    lo = n - 2048
    tr = tuple(t[lo:] for t in lay.tracks())
    q, k, v = (case.full[i][lo:].cpu() for i in range(3))
    o_ref, lse_ref = oatt.forward_rows(tr, w, q, k, v, sel - lo, 1.0 / np.sqrt(lay.d))
    tsel = torch.from_numpy(sel).cuda()
    eo = max_err(o[tsel].float().cpu().numpy(), o_ref)
    el = max_err(lse[:, tsel].cpu().numpy(), lse_ref)
    print(f"  rows past 2 GiB of K/V: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= O_TOL and el <= LSE_TOL
