"""GPU parity of the backward ring steps against the fp64 oracle gradients."""
import numpy as np
import pytest
import torch

import block_sparse_masked_metadata_amd as bsm
from workloads import random_small, sliding_window, long_mixed, packed_multimodal
from oracle import backward as obwd
from gpu_common import Case, check_rows, grad_ok, needs_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not needs_gpu, reason="needs a GPU")]


def _run(case):
    o, lse, _ = case.ring()
    dq, dks, dvs = bsm.bwd_ring(case.dp, case.heads, case.q, case.k_shards, case.v_shards,
                                case.dout, o, lse)
    torch.cuda.synchronize()
    return o, lse, dq, dks, dvs


def _oracle(case, sel):
    return obwd.backward_rows(case.lay.tracks(), case.lay.window, case.cpu(0), case.cpu(1),
                              case.cpu(2), case.cpu(3), case.rows[sel], 1.0 / np.sqrt(case.lay.d))


def _check_full(case):
    """All of the rank's rows: dQ, and dK/dV of every key (zero where unread)."""
    o, lse, dq, dks, dvs = _run(case)
    sel = np.arange(case.S)
    ref = _oracle(case, sel)
    e1 = grad_ok(dq.cpu().numpy(), ref["dq"], "dq")
    n, hkv, d = case.lay.n, case.hkv, 128
    dk = np.zeros((n, hkv, d))
    dv = np.zeros((n, hkv, d))
    dk[case.perm] = torch.cat(dks).cpu().numpy()
    dv[case.perm] = torch.cat(dvs).cpu().numpy()
    dk_ref = np.zeros_like(dk)
    dv_ref = np.zeros_like(dv)
    for a, b, dkb, dvb in ref["dkv"]:
        dk_ref[a:b] += dkb
        dv_ref[a:b] += dvb
    e2 = grad_ok(dk, dk_ref, "dk")
    e3 = grad_ok(dv, dv_ref, "dv")
    print(f"  dq {e1:.3e} dk {e2:.3e} dv {e3:.3e}", flush=True)


@pytest.mark.parametrize("seed", range(4))
def test_random_layouts_backward(seed):
    rng = np.random.default_rng(700 + seed)
    ranks = [2, 4, 3, 1][seed]
    order = ["ptrr", "contiguous"][seed % 2]
    n = 128 * ranks * [2, 1, 2, 3][seed]
    lay = random_small(rng, n, max_span=300)
    lay.ranks, lay.order, lay.seed = ranks, order, 60 + seed
    lay.hq, lay.hkv, lay.d = [(4, 2), (2, 2), (6, 3), (4, 1)][seed] + (128,)
    for r in range(ranks):
        _check_full(Case(lay, rank=r, with_do=True))


@pytest.mark.parametrize("seed", range(4))
def test_ragged_shards_forward_and_backward(seed):
    """Shards that are not multiples of 128 rows: the last tile of every shard
    is ragged, and with S % 128 <= 64 its second 64-row half has no valid row
    (the sub-tile the kernels stage as zeros by the record count).  O/LSE,
    dQ and dK/dV of every rank against the oracle, several GQA ratios."""
    rng = np.random.default_rng(1700 + seed)
    ranks = [2, 3, 1, 4][seed]
    S = [164, 100, 37, 230][seed]
    lay = random_small(rng, S * ranks, max_span=120)
    lay.ranks, lay.order, lay.seed = ranks, "contiguous", 80 + seed  # block orders need whole blocks
    lay.hq, lay.hkv, lay.d = [(4, 2), (3, 1), (2, 2), (8, 4)][seed] + (128,)
    for r in range(ranks):
        case = Case(lay, rank=r, with_do=True)
        assert case.S == S
        o, lse, _ = case.ring()
        torch.cuda.synchronize()
        check_rows(case, o, lse)
        _check_full(case)


def test_sliding_window_scaled_full_backward():
    """Same recipe as the 128K sliding-window layer at 1/8 size (clip 2048, W 512)."""
    lay = sliding_window(n=16384, clip=2048, window=512)
    _check_full(Case(lay, with_do=True))


def test_packed_multimodal_scaled_full_backward():
    lay = packed_multimodal(n=8192, seed=3)
    lay.hq = lay.hkv = 4
    _check_full(Case(lay, with_do=True))


def _check_key_sums(case, o, lse, dks, dvs):
    """Sums over every key of the rank's dK/dV, which hold at any size.

    Rows of P sum to 1, so the sum over keys of dV equals the sum over the
    rank's queries of dO (per key/value head: the group's query heads added).
    The kernels round P to bf16 (relative error at most 2^-9 per term), so the
    two sides differ by at most 2^-9 sum |dO| per channel; the test allows 2^-8.

    Sum_j dS_ij = sum_j P_ij (dP_ij - D_i) = dO_i . (O_exact_i - O_i) plus the
    bf16 rounding of P and dS, so sum over keys of dK = scale sum_i q_i sum_j
    dS_ij is zero up to E_i = 2^-7 (|dO_i|_2 Vmax + |D_i|) per query and head,
    Vmax the largest |v_j|_2 of the head: |O_exact - O| <= 2^-8 Vmax (bf16 O
    and bf16 P), the dS rounding adds 2^-9 (|dO_i|_2 Vmax + |D_i|).  A wrong
    D, LSE, scale or a dropped key tile moves either sum by orders of magnitude
    more than these bounds."""
    grp = case.hq // case.hkv
    live = torch.isfinite(lse).T[:, :, None]                      # [S, hq, 1]: rows with a legal key
    do = torch.where(live, case.dout.double(), torch.zeros((), dtype=torch.float64, device="cuda"))
    dv_sum = sum(d.double().sum(0) for d in dvs)                  # [hkv, d]
    do_sum = do.sum(0).view(case.hkv, grp, -1).sum(1)
    do_abs = do.abs().sum(0).view(case.hkv, grp, -1).sum(1)
    err_v = ((dv_sum - do_sum).abs() / do_abs.clamp_min(1e-30)).max().item()
    assert err_v <= 2.0 ** -8, f"sum of dV over keys: relative error {err_v:.3e}"
    scale = 1.0 / np.sqrt(case.lay.d)
    vmax = case.v_all.double().norm(dim=2).max(0).values          # [hkv]
    vmax_q = vmax.repeat_interleave(grp)[None, :]                   # [1, hq]
    dd = (do * o.double()).sum(2)                                   # D_i per head [S, hq]
    e = 2.0 ** -7 * (do.norm(dim=2) * vmax_q + dd.abs())            # [S, hq]
    bound = scale * (case.q.double().abs() * e[:, :, None]).sum(0).view(case.hkv, grp, -1).sum(1)
    dk_sum = sum(d.double().sum(0) for d in dks)
    ratio = (dk_sum.abs() / bound.clamp_min(1e-30)).max().item()
    assert ratio <= 1.0, f"sum of dK over keys exceeds its rounding bound ({ratio:.3f} of it)"
    print(f"  key sums: dV rel {err_v:.3e}, dK at {ratio:.3e} of its bound", flush=True)


@pytest.mark.parametrize("maker", [sliding_window, long_mixed], ids=["sliding_window_128k", "long_mixed_1m"])
def test_full_size_dq_sampled(maker):
    case = Case(maker(), with_do=True)
    o, lse, dq, dks, dvs = _run(case)
    _check_key_sums(case, o, lse, dks, dvs)
    rng = np.random.default_rng(3)
    sel = np.sort(rng.choice(case.S, 128, replace=False))
    ref = _oracle(case, sel)
    e = grad_ok(dq[torch.from_numpy(sel).cuda()].cpu().numpy(), ref["dq"], "dq")
    print(f"  dq sampled {e:.3e}", flush=True)
    # dK/dV only where the rank's queries can read: everything else stays 0
    for j in range(case.R):
        if case.dp.info["bwd_items"][(case.r - j) % case.R] == 0:
            assert torch.count_nonzero(dks[j]) == 0 and torch.count_nonzero(dvs[j]) == 0


def test_split_dkdv_matches_unsplit_and_oracle():
    """Packed text: the dK/dV launch has fewer (key tile, kv head) units than
    twice the CUs, so with a workspace its long column lists are split and
    reduced in order.  Split and unsplit gradients both match the oracle and
    each other to rounding."""
    from workloads import packed_text
    case = Case(packed_text(), with_do=True)
    assert case.dp.info["bwd_workspace_slots"] > 0
    o, lse, _ = case.ring()
    g_split = bsm.bwd_ring(case.dp, case.heads, case.q, case.k_shards, case.v_shards, case.dout, o, lse,
                           split=True)
    g_plain = bsm.bwd_ring(case.dp, case.heads, case.q, case.k_shards, case.v_shards, case.dout, o, lse,
                           split=False)
    torch.cuda.synchronize()
    for x, y in zip([g_split[0]] + g_split[1] + g_split[2], [g_plain[0]] + g_plain[1] + g_plain[2]):
        assert float((x - y).abs().max()) <= 1e-3 * max(1.0, float(y.abs().max()))
    sel = np.arange(case.S)
    ref = _oracle(case, sel)
    grad_ok(g_split[0].cpu().numpy(), ref["dq"], "dq")
    n, hkv = case.lay.n, case.hkv
    dk = np.zeros((n, hkv, 128))
    dv = np.zeros_like(dk)
    dk[case.perm] = torch.cat(g_split[1]).cpu().numpy()
    dv[case.perm] = torch.cat(g_split[2]).cpu().numpy()
    dk_ref = np.zeros_like(dk)
    dv_ref = np.zeros_like(dv)
    for a, b, dkb, dvb in ref["dkv"]:
        dk_ref[a:b] += dkb
        dv_ref[a:b] += dvb
    e2 = grad_ok(dk, dk_ref, "dk")
    e3 = grad_ok(dv, dv_ref, "dv")
    print(f"  split dk {e2:.3e} dv {e3:.3e}", flush=True)


def test_split_workspace_too_small_is_refused():
    """Every buffer is real and sized for the step, so the call is a valid
    launch whether or not the step splits; a step that splits must refuse a
    16-byte workspace before launching."""
    from workloads import packed_text
    case = Case(packed_text(), with_do=True)
    o, lse, _ = case.ring()
    delta = bsm.bwd_prep(case.heads, o, case.dout)
    dq = torch.zeros(case.S, case.hq, 128, dtype=torch.float32, device="cuda")
    dk = torch.zeros(case.S, case.hkv, 128, dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    tiny = torch.zeros(4, dtype=torch.float32, device="cuda")
    refused = 0
    for s in range(case.R):
        j = (case.r - s) % case.R
        try:
            bsm.bwd_step(case.dp, s, case.heads, case.q, case.k_shards[j], case.v_shards[j], case.dout,
                         lse, delta, dq, dk, dv, workspace=tiny)
        except bsm.BsmError as e:
            assert e.code == bsm._capi.BSM_E_INVALID and "workspace" in str(e)
            refused += 1
    torch.cuda.synchronize()
    assert refused > 0


@pytest.mark.parametrize("maker", ["packed_text", "random"])
def test_two_streams_equal_one_stream(maker):
    """bsm_bwd_step_streams: the dK/dV chain on a second stream, or its
    launches alternating over two side streams, gives the one-stream
    gradients bit for bit (same kernels, same inputs)."""
    from workloads import packed_text
    if maker == "packed_text":
        lay = packed_text()
    else:
        rng = np.random.default_rng(91)
        lay = random_small(rng, 128 * 4 * 2, max_span=300)
        lay.ranks, lay.order, lay.seed = 4, "ptrr", 17
        lay.hq, lay.hkv, lay.d = 4, 2, 128
    case = Case(lay, with_do=True)
    o, lse, _ = case.ring()
    one = bsm.bwd_ring(case.dp, case.heads, case.q, case.k_shards, case.v_shards, case.dout, o, lse,
                       two_streams=False)
    two = bsm.bwd_ring(case.dp, case.heads, case.q, case.k_shards, case.v_shards, case.dout, o, lse,
                       two_streams=True, kv_streams=1)
    # dK/dV launches of successive steps alternating over two side streams
    three = bsm.bwd_ring(case.dp, case.heads, case.q, case.k_shards, case.v_shards, case.dout, o, lse,
                         two_streams=True, kv_streams=2)
    torch.cuda.synchronize()
    for other in (two, three):
        assert torch.equal(one[0], other[0])
        for a, b in zip(one[1] + one[2], other[1] + other[2]):
            assert torch.equal(a, b)
    if maker == "random":
        sel = np.arange(case.S)
        ref = _oracle(case, sel)
        grad_ok(two[0].cpu().numpy(), ref["dq"], "dq")


def _offset_view(t, nbytes):
    """A copy of `t` whose data pointer sits `nbytes` past a 256-byte boundary."""
    elems = nbytes // t.element_size()
    buf = torch.empty(t.numel() + elems, dtype=t.dtype, device=t.device)
    v = buf[elems:elems + t.numel()].view(t.shape)
    v.copy_(t)
    return v


def test_misaligned_tensors_are_refused():
    """A tensor pointer 8 bytes off its 16-byte alignment returns BSM_E_INVALID
    from the forward and the backward step before anything is launched: the
    outputs keep their contents."""
    rng = np.random.default_rng(5)
    lay = random_small(rng, 128 * 2 * 2, max_span=200)
    lay.ranks, lay.order, lay.seed = 2, "ptrr", 3
    lay.hq, lay.hkv, lay.d = 2, 2, 128
    case = Case(lay, with_do=True)
    q_bad = _offset_view(case.q, 8)
    assert q_bad.data_ptr() % 16 == 8
    state = bsm.new_state(case.S, case.hq, 128)
    o = torch.full((case.S, case.hq, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((case.hq, case.S), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(bsm.BsmError) as err:
        bsm.fwd_step(case.dp, 0, case.heads, q_bad, case.k_shards[case.r], case.v_shards[case.r], state, o, lse)
    assert err.value.code == bsm._capi.BSM_E_INVALID and "16-byte" in str(err.value)
    o_ok, lse_ok, _ = case.ring()
    delta = bsm.bwd_prep(case.heads, o_ok, case.dout)
    dq = torch.full((case.S, case.hq, 128), 7.0, dtype=torch.float32, device="cuda")
    dq_bad = _offset_view(dq, 8)
    dk = torch.zeros(case.S, case.hkv, 128, dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    with pytest.raises(bsm.BsmError) as err:
        bsm.bwd_step(case.dp, 0, case.heads, case.q, case.k_shards[case.r], case.v_shards[case.r], case.dout,
                     lse_ok, delta, dq_bad, dk, dv)
    assert err.value.code == bsm._capi.BSM_E_INVALID
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all()) and bool((dq_bad == 7.0).all())
    assert torch.count_nonzero(dk) == 0 and torch.count_nonzero(dv) == 0
