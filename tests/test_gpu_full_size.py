"""Full-size parity of the two forward + backward workloads, element by element
against the fp64 oracle (MARBLE section 05 "Accuracy": outputs and gradients
against a whole-sequence reference; section 03: the ring's fp32 carry gives
one GPU's result exactly).

- Sliding window 128K (8 clips of 16384 tokens, W = 4096, Hq/Hkv = 16/4): the
  busiest rank's whole share, 16,384 query rows: O (pre-rounding and bf16),
  LSE, dQ of every row, dK and dV of every key of the rank's sample.
- Long mixed 1M (Hq/Hkv = 16/4): whole samples of the busiest rank's share,
  its 3 clips with the most rows there plus 50 random text documents: every
  row of the rank in those samples, and dK/dV of every key of those samples.
  No sample attends another, so this subset is exact: a key's gradient comes
  only from queries of its own sample.

Both also check that the ring equals the single pass bit for bit, and that
dK/dV of keys the rank's queries cannot read stay exactly zero.
"""
import time

import numpy as np
import pytest
import torch

import block_sparse_masked_metadata_amd as bsm
from workloads import sliding_window, long_mixed
from oracle import backward as obwd
from gpu_common import Case, O_TOL, LSE_TOL, GRAD_REL, max_err, needs_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not needs_gpu, reason="needs a GPU")]


def _run_gpu(case):
    """Ring forward (bf16 O, LSE; and the pre-rounding fp32 state), the single
    pass, and the ring backward (two streams, split dK/dV work as the bench)."""
    _, _, st_ring = case.ring(keep_state=True)
    st_single = case.single(keep_state=True)
    o, lse, _ = case.ring()
    o1, l1 = case.single()
    torch.cuda.synchronize()
    for a, b in zip(st_ring, st_single):
        assert torch.equal(a, b), "ring state differs from the single pass"
    assert torch.equal(o, o1) and torch.equal(lse, l1), "ring O/LSE differ from the single pass"
    del st_single, o1, l1
    dq, dks, dvs = bsm.bwd_ring(case.dp, case.heads, case.q, case.k_shards, case.v_shards,
                                case.dout, o, lse)
    torch.cuda.synchronize()
    return o, lse, st_ring, dq, dks, dvs


def _compare(case, sel, ref, o, lse, st, dq, dks, dvs):
    """sel: indices into the rank's shard; ref: oracle.backward_rows of case.rows[sel]."""
    tsel = torch.from_numpy(sel).cuda()
    acc, _, l = st
    acc = bsm.state_rows(case.heads, acc, case.S)[tsel]
    lt = l[:, tsel].T[:, :, None]
    o32 = acc * torch.where(lt > 0, 1.0 / torch.where(lt > 0, lt, torch.ones_like(lt)), torch.zeros_like(lt))
    og = o[tsel]
    assert torch.equal(og, o32.to(torch.bfloat16)), "bf16 O is not RNE(O_acc * (1 / l))"
    eo = max_err(o32.cpu().numpy(), ref["o"])
    el = max_err(lse[:, tsel].cpu().numpy(), ref["lse"])
    assert eo <= O_TOL and el <= LSE_TOL, (eo, el)
    dq_ref = ref["dq"]
    edq = float(np.abs(dq[tsel].cpu().numpy() - dq_ref).max())
    tol_q = GRAD_REL * max(1.0, float(np.abs(dq_ref).max()))
    assert edq <= tol_q, f"dq: {edq:.3e} > {tol_q:.3e}"
    # dK/dV of every key of the samples the oracle covered, gathered from the
    # shards (plan order) by original index
    inv = np.empty(case.lay.n, np.int64)
    inv[case.perm] = np.arange(case.lay.n)
    dk_all = torch.cat(dks)
    dv_all = torch.cat(dvs)
    edk = edv = 0.0
    mk = mv = 1.0
    seen = np.zeros(case.lay.n, bool)
    for a, b, dkb, dvb in ref["dkv"]:
        idx = torch.from_numpy(inv[a:b]).cuda()
        gk = dk_all.index_select(0, idx).cpu().numpy()
        gv = dv_all.index_select(0, idx).cpu().numpy()
        edk = max(edk, float(np.abs(gk - dkb).max()))
        edv = max(edv, float(np.abs(gv - dvb).max()))
        mk = max(mk, float(np.abs(dkb).max()))
        mv = max(mv, float(np.abs(dvb).max()))
        seen[a:b] = True
    assert edk <= GRAD_REL * mk, f"dk: {edk:.3e} > {GRAD_REL * mk:.3e}"
    assert edv <= GRAD_REL * mv, f"dv: {edv:.3e} > {GRAD_REL * mv:.3e}"
    print(f"  rows={len(sel)} keys={int(seen.sum())} |dO32|={eo:.3e} |dLSE|={el:.3e} "
          f"|ddQ|={edq:.3e} |ddK|={edk:.3e} |ddV|={edv:.3e}", flush=True)
    return seen


def _oracle(case, sel):
    t0 = time.perf_counter()
    ref = obwd.backward_rows(case.lay.tracks(), case.lay.window, case.cpu(0), case.cpu(1),
                             case.cpu(2), case.cpu(3), case.rows[sel], 1.0 / np.sqrt(case.lay.d))
    print(f"  oracle: {len(sel)} rows in {time.perf_counter() - t0:.1f} s", flush=True)
    return ref


def test_sliding_window_128k_full_share():
    case = Case(sliding_window(), with_do=True)
    out = _run_gpu(case)
    sel = np.arange(case.S)
    seen = _compare(case, sel, _oracle(case, sel), *out)
    # every key outside the rank's sample has zero gradient
    inv = np.empty(case.lay.n, np.int64)
    inv[case.perm] = np.arange(case.lay.n)
    other = torch.from_numpy(inv[~seen]).cuda()
    dks, dvs = out[4], out[5]
    assert torch.count_nonzero(torch.cat(dks).index_select(0, other)) == 0
    assert torch.count_nonzero(torch.cat(dvs).index_select(0, other)) == 0


def _long_mixed_samples(case, clips=3, texts=50, seed=5):
    """The rank's rows in its `clips` clip samples with the most rows there and
    in `texts` random text documents (shard indices)."""
    sample = case.lay.sample
    mine = sample[case.rows]
    sid, nrows = np.unique(mine, return_counts=True)
    is_clip = case.lay.seg[case.rows] >= 0            # a clip is one bidirectional span
    clip_set = set(np.unique(mine[is_clip]).tolist())
    clip_ids = [int(s) for s in sid if int(s) in clip_set]
    text_ids = [int(s) for s in sid if int(s) not in clip_set]
    rows_of = dict(zip(sid.tolist(), nrows.tolist()))
    clip_ids.sort(key=lambda s: (-rows_of[s], s))
    rng = np.random.default_rng(seed)
    pick = clip_ids[:clips] + sorted(rng.choice(text_ids, texts, replace=False).tolist())
    return np.flatnonzero(np.isin(mine, pick)), pick


def test_long_mixed_1m_whole_samples():
    case = Case(long_mixed(), with_do=True)
    out = _run_gpu(case)
    sel, pick = _long_mixed_samples(case)
    assert len(pick) == 53
    _compare(case, sel, _oracle(case, sel), *out)
    # shards the rank never reads keep zero dK/dV
    dks, dvs = out[4], out[5]
    for j in range(case.R):
        if case.dp.info["bwd_items"][(case.r - j) % case.R] == 0:
            assert torch.count_nonzero(dks[j]) == 0 and torch.count_nonzero(dvs[j]) == 0
