"""Torch-facing helpers over the C ABI: plans, device plans and the step loops.

Argument marshalling and orchestration only.  Every step of the path runs in
libbsm's kernels; PyTorch provides device memory (caller-owned buffers) and the
current HIP stream.  Layouts follow include/bsm.h.
"""
from __future__ import annotations

import math

import numpy as np

from . import _capi as C


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous {dtype} cuda tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")


class Plan:
    """Host plan (owned handle).  `tracks` = (sample, seg, noise, pos) in original order."""

    def __init__(self, tracks, window, ranks, block=128, order="ptrr", explicit_block_perm=None,
                 threads=0):
        self.handle = C.bsm_plan_build(*tracks, window, ranks, block, C.ORDERS[order],
                                       explicit_block_perm, threads)
        self.info = C.bsm_plan_get_info(self.handle)

    @classmethod
    def from_layout(cls, layout, threads=0):
        return cls(layout.tracks(), layout.window, layout.ranks, layout.block, layout.order,
                   explicit_block_perm=getattr(layout, "block_perm", None), threads=threads)

    def permutation(self):
        return C.bsm_plan_permutation(self.handle)

    def step_map(self, r, s):
        return C.bsm_plan_step_map(self.handle, r, s)

    def pairs(self):
        return C.bsm_plan_pairs(self.handle)

    def block_cost(self):
        return C.bsm_plan_block_cost(self.handle)

    def chunk_order(self, min_chunks=1, max_chunks=64, tau=0.0, swaps=4):
        """Chunked ring layout: (explicit block order, cost terms)."""
        return C.bsm_plan_chunk_order(self.handle, min_chunks, max_chunks, tau, swaps)

    def dense_calls(self, r, s):
        """int32 [count, 5] (q0, q_len, k0, k_len, kind): rank r's dense calls at step s."""
        return C.bsm_plan_dense_calls(self.handle, r, s)

    def fetch_set(self, r):
        """(needed [R, tiles_per_shard] uint8, count): remote key tiles rank r needs."""
        return C.bsm_plan_fetch_set(self.handle, r)

    def key_intervals(self):
        """(lo, hi) per key in the original order; hi < lo: no single range."""
        return C.bsm_plan_key_intervals(self.handle)

    def close(self):
        if self.handle:
            C.bsm_plan_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def vision_group_order(tracks):
    """The vision-group layout transform: new_to_orig over the tokens of
    `tracks` (sample, seg, noise, pos), to be applied to tracks and
    activations alike before planning."""
    return C.bsm_vision_group_order(tracks[0], tracks[1])


class DevicePlan:
    """Rank r's device plan in a torch uint8 buffer (the library allocates nothing)."""

    def __init__(self, plan: Plan, r: int, device="cuda", dense=False):
        """dense: forward lists from the plan's dense calls (forward steps and
        the single pass only)."""
        import torch
        nbytes = (C.bsm_dplan_calls_bytes if dense else C.bsm_dplan_bytes)(plan.handle, r)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        upload = C.bsm_dplan_calls_upload if dense else C.bsm_dplan_upload
        self.handle = upload(plan.handle, r, self.buf.data_ptr(), nbytes, _stream())
        self.info = C.bsm_dplan_get_info(self.handle)
        self.rank = r
        self.ranks = plan.info["ranks"]
        self.rows = plan.info["shard_tokens"]

    def close(self):
        if self.handle:
            C.bsm_dplan_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def heads(hq, hkv, d=128, scale=None):
    return C._heads(hq, hkv, d, 1.0 / math.sqrt(d) if scale is None else scale)


def new_state(rows, hq, d, device="cuda"):
    """Uninitialized fp32 state (O_acc, m, l): the first step initializes it in-kernel.
    O_acc is the kernels' tile-blocked buffer (flat, ceil(rows/128)*128*hq*d
    floats); state_rows reads it out in row order."""
    import torch
    padded = (rows + 127) // 128 * 128
    return (torch.empty(padded * hq * d, dtype=torch.float32, device=device),
            torch.empty(hq, rows, dtype=torch.float32, device=device),
            torch.empty(hq, rows, dtype=torch.float32, device=device))


def state_rows(hd, o_acc, rows):
    """The tile-blocked O_acc as fp32 [rows, Hq, d]."""
    import torch
    _need(o_acc, torch.float32, ((rows + 127) // 128 * 128 * hd.hq * hd.d,), "o_acc")
    out = torch.empty(rows, hd.hq, hd.d, dtype=torch.float32, device=o_acc.device)
    C.bsm_state_unpack(hd, rows, _ptr(o_acc), _ptr(out), _stream())
    return out


def fwd_step(dp: DevicePlan, s, hd, q, k, v, state, o, lse, keep_state=False, chain=None):
    """One forward ring step on the current stream: every query tile with work
    (bsm_fwd_step), or with chain 0 or 1 only that chain's tiles
    (bsm_fwd_step_chain)."""
    o_acc, m, l = state
    flags = C.BSM_FWD_KEEP_STATE if keep_state else 0
    if chain is None:
        C.bsm_fwd_step(dp.handle, s, hd, _ptr(q), _ptr(k), _ptr(v), _ptr(o_acc), _ptr(m), _ptr(l),
                       _ptr(o), _ptr(lse), flags, _stream())
    else:
        C.bsm_fwd_step_chain(dp.handle, s, chain, hd, _ptr(q), _ptr(k), _ptr(v), _ptr(o_acc), _ptr(m),
                             _ptr(l), _ptr(o), _ptr(lse), flags, _stream())


CHAIN_MAX_ROUNDS = 8


def fwd_chains(dp: DevicePlan, hd, device=None):
    """How many chains the forward ring should run (bsm_fwd_step_chain): 2
    when at every step with work each chain holds at least one full round of
    workgroups (two per CU) and at most CHAIN_MAX_ROUNDS, so that each chain's
    launches fill the chip and the other chain's launches fill their tails;
    else 1.  Below a round per chain the two half launches leave CUs idle
    (packed text 32K was 7-8% slower with two chains); over many rounds a
    launch's tail is a small part of it and the second chain only contends
    (long mixed 1M, 32 rounds per launch: 0.7% slower)."""
    import torch
    full = 2 * torch.cuda.get_device_properties(device if device is not None else
                                                torch.cuda.current_device()).multi_processor_count
    work = False
    for s in range(dp.ranks):
        n, c0 = dp.info["fwd_items"][s], dp.info["fwd_chain0_items"][s]
        if n == 0:
            continue
        work = True
        if min(c0, n - c0) * hd.hq < full or max(c0, n - c0) * hd.hq > CHAIN_MAX_ROUNDS * full:
            return 1
    return 2 if work else 1


def fwd_ring(dp: DevicePlan, hd, q, k_shards, v_shards, state=None, out=None, keep_state=False,
             steps=None, chains=None):
    """Run ring steps s = 0..R-1 (shard j = (r - s) mod R from k_shards[j]).

    chains: 1 runs every step in one launch on the current stream; 2 runs the
    plan's two chains of query tiles on two side streams, each chain's steps
    in order (bitwise the same result); None picks fwd_chains(dp, hd).  The
    side streams wait for the current stream first and the current stream
    waits for them before returning.  Returns (o, lse, state)."""
    import torch
    rows = dp.rows
    _need(q, torch.bfloat16, (rows, hd.hq, hd.d), "q")
    for j in range(dp.ranks):
        _need(k_shards[j], torch.bfloat16, (rows, hd.hkv, hd.d), f"k_shards[{j}]")
        _need(v_shards[j], torch.bfloat16, (rows, hd.hkv, hd.d), f"v_shards[{j}]")
    if state is None:
        state = new_state(rows, hd.hq, hd.d, q.device)
    if out is None:
        out = (torch.empty(rows, hd.hq, hd.d, dtype=torch.bfloat16, device=q.device),
               torch.empty(hd.hq, rows, dtype=torch.float32, device=q.device))
    o, lse = out
    todo = list(range(dp.ranks) if steps is None else steps)
    nch = fwd_chains(dp, hd, q.device) if chains is None else int(chains)
    if nch not in (1, 2):
        raise ValueError(f"chains: expected 1 or 2, got {chains}")
    if nch == 1:
        for s in todo:
            j = (dp.rank - s) % dp.ranks
            fwd_step(dp, s, hd, q, k_shards[j], v_shards[j], state, o, lse, keep_state)
        return o, lse, state
    main = torch.cuda.current_stream()
    sides = _side_streams(q.device, 2)
    for side in sides:
        side.wait_stream(main)
    for s in todo:
        j = (dp.rank - s) % dp.ranks
        for c, side in enumerate(sides):
            with torch.cuda.stream(side):
                fwd_step(dp, s, hd, q, k_shards[j], v_shards[j], state, o, lse, keep_state, chain=c)
    for side in sides:
        main.wait_stream(side)
    return o, lse, state


def fwd_ring_merged(dp: DevicePlan, hd, q, k_shards, v_shards, mode="bf16", steps=None):
    """Accuracy controls: each ring step finishes its own keys (BSM_FWD_STEP_ONLY)
    and is merged into a running result, instead of carrying (O_acc, m, l).

    mode "bf16": per-step normalized bf16 O_s and LSE_s, merged into a bf16 O.
    mode "fp32": per-step unnormalized fp32 partials, merged into an fp32 O.
    Returns (o bf16 [S, Hq, d], lse fp32 [Hq, S])."""
    import torch
    rows, dev = dp.rows, q.device
    shape = (rows, hd.hq, hd.d)
    lse_run = torch.full((hd.hq, rows), -math.inf, dtype=torch.float32, device=dev)
    acc, m, l = new_state(rows, hd.hq, hd.d, dev)
    todo = [s for s in (range(dp.ranks) if steps is None else steps) if dp.info["fwd_items"][s] > 0]
    if mode == "bf16":
        o_run = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
        o_s = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        lse_s = torch.empty(hd.hq, rows, dtype=torch.float32, device=dev)
        for s in todo:
            j = (dp.rank - s) % dp.ranks
            lse_s.fill_(-math.inf)  # rows this step does not reach
            C.bsm_fwd_step(dp.handle, s, hd, _ptr(q), _ptr(k_shards[j]), _ptr(v_shards[j]), _ptr(acc),
                           _ptr(m), _ptr(l), _ptr(o_s), _ptr(lse_s), C.BSM_FWD_STEP_ONLY, _stream())
            C.bsm_fwd_merge_bf16(hd, rows, _ptr(o_run), _ptr(lse_run), _ptr(o_s), _ptr(lse_s), _stream())
        return o_run, lse_run
    if mode != "fp32":
        raise ValueError("mode must be 'bf16' or 'fp32'")
    o_run = torch.zeros(shape, dtype=torch.float32, device=dev)
    o = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    for i, s in enumerate(todo):
        j = (dp.rank - s) % dp.ranks
        l.fill_(0.0)  # rows this step does not reach
        C.bsm_fwd_step(dp.handle, s, hd, _ptr(q), _ptr(k_shards[j]), _ptr(v_shards[j]), _ptr(acc), _ptr(m),
                       _ptr(l), None, None, C.BSM_FWD_STEP_ONLY | C.BSM_FWD_KEEP_STATE, _stream())
        C.bsm_fwd_merge_fp32(hd, rows, _ptr(o_run), _ptr(lse_run), _ptr(acc), _ptr(m), _ptr(l),
                             _ptr(o) if i == len(todo) - 1 else None, _stream())
    return o, lse_run


def fetch_rows(plan: Plan, r: int):
    """Source row (into the shards concatenated in plan order) of every row of
    rank r's compact sparse-fetch buffer: its own shard, then each needed
    remote tile (128 rows, ring step order, ascending tile); -1 pads a ragged
    tile."""
    need, _ = plan.fetch_set(r)
    R, T = need.shape
    S = plan.info["shard_tokens"]
    out = [np.arange(r * S, (r + 1) * S, dtype=np.int64)]
    for s in range(1, R):
        j = (r - s) % R
        for b in np.flatnonzero(need[j]):
            src = np.arange(j * S + b * 128, j * S + b * 128 + 128, dtype=np.int64)
            src[src >= (j + 1) * S] = -1
            out.append(src)
    return np.concatenate(out)


def gather_fetched(plan: Plan, r: int, k_all, v_all):
    """The compact key/value buffers of rank r from all shards (what one
    variable-sized all-to-all would deliver); pad rows copy row 0."""
    import torch
    src = torch.from_numpy(np.maximum(fetch_rows(plan, r), 0)).to(k_all.device)
    return k_all.index_select(0, src), v_all.index_select(0, src)


def fwd_fetched(dp: DevicePlan, hd, q, k_fetch, v_fetch, out=None, keep_state=False):
    """One pass over the rank's shard and its fetched remote tiles.
    keep_state: return the unnormalized state (O_acc, m, l) instead of (o, lse)."""
    import torch
    rows = dp.rows
    _need(q, torch.bfloat16, (rows, hd.hq, hd.d), "q")
    fr = dp.info["fetch_rows"]
    _need(k_fetch, torch.bfloat16, (fr, hd.hkv, hd.d), "k_fetch")
    _need(v_fetch, torch.bfloat16, (fr, hd.hkv, hd.d), "v_fetch")
    if keep_state:
        state = new_state(rows, hd.hq, hd.d, q.device)
        C.bsm_fwd_fetched(dp.handle, hd, _ptr(q), _ptr(k_fetch), _ptr(v_fetch), *(_ptr(t) for t in state),
                          None, None, C.BSM_FWD_KEEP_STATE, _stream())
        return state
    if out is None:
        out = (torch.empty(rows, hd.hq, hd.d, dtype=torch.bfloat16, device=q.device),
               torch.empty(hd.hq, rows, dtype=torch.float32, device=q.device))
    o, lse = out
    C.bsm_fwd_fetched(dp.handle, hd, _ptr(q), _ptr(k_fetch), _ptr(v_fetch), None, None, None, _ptr(o),
                      _ptr(lse), 0, _stream())
    return o, lse


def bwd_fetched(dp: DevicePlan, hd, q, k_fetch, v_fetch, dout, o, lse):
    """Backward of the sparse-fetch pass: (dq, dk_fetch, dv_fetch) in fp32,
    dk/dv over the rows of the compact buffer (the rank's contributions, to be
    sent back to the owners: fetched_accumulate)."""
    import torch
    rows = dp.rows
    _need(dout, torch.bfloat16, (rows, hd.hq, hd.d), "dout")
    fr = dp.info["fetch_rows"]
    _need(k_fetch, torch.bfloat16, (fr, hd.hkv, hd.d), "k_fetch")
    _need(v_fetch, torch.bfloat16, (fr, hd.hkv, hd.d), "v_fetch")
    delta = bwd_prep(hd, o, dout)
    dq = torch.empty(rows, hd.hq, hd.d, dtype=torch.float32, device=q.device)
    dkf = torch.zeros(fr, hd.hkv, hd.d, dtype=torch.float32, device=q.device)
    dvf = torch.zeros_like(dkf)
    C.bsm_bwd_fetched(dp.handle, hd, _ptr(q), _ptr(k_fetch), _ptr(v_fetch), _ptr(dout), _ptr(lse), _ptr(delta),
                      _ptr(dq), _ptr(dkf), _ptr(dvf), _stream())
    return dq, dkf, dvf


def fetched_accumulate(dp: DevicePlan, hd, dk_fetch, dv_fetch, dk_all, dv_all):
    """dk_all/dv_all (fp32, all shards in plan order) += the compact rows'
    contributions at their shard rows (the sparse fetch's way back)."""
    import torch
    fr = dp.info["fetch_rows"]
    for t, name in ((dk_fetch, "dk_fetch"), (dv_fetch, "dv_fetch")):
        _need(t, torch.float32, (fr, hd.hkv, hd.d), name)
    for t, name in ((dk_all, "dk_all"), (dv_all, "dv_all")):
        _need(t, torch.float32, (dp.rows * dp.ranks, hd.hkv, hd.d), name)
    C.bsm_fetched_accumulate(dp.handle, hd, _ptr(dk_fetch), _ptr(dv_fetch), _ptr(dk_all), _ptr(dv_all), _stream())


def fwd_single(dp: DevicePlan, hd, q, k_all, v_all, keep_state=False, out=None):
    """Single pass over all shards (k_all/v_all = shards concatenated in plan order)."""
    import torch
    rows = dp.rows
    _need(q, torch.bfloat16, (rows, hd.hq, hd.d), "q")
    _need(k_all, torch.bfloat16, (rows * dp.ranks, hd.hkv, hd.d), "k_all")
    _need(v_all, torch.bfloat16, (rows * dp.ranks, hd.hkv, hd.d), "v_all")
    if keep_state:
        state = new_state(rows, hd.hq, hd.d, q.device)
        C.bsm_fwd_single(dp.handle, hd, _ptr(q), _ptr(k_all), _ptr(v_all), *(_ptr(t) for t in state),
                         None, None, C.BSM_FWD_KEEP_STATE, _stream())
        return state
    if out is None:
        out = (torch.empty(rows, hd.hq, hd.d, dtype=torch.bfloat16, device=q.device),
               torch.empty(hd.hq, rows, dtype=torch.float32, device=q.device))
    o, lse = out
    C.bsm_fwd_single(dp.handle, hd, _ptr(q), _ptr(k_all), _ptr(v_all), None, None, None,
                     _ptr(o), _ptr(lse), 0, _stream())
    return o, lse


def bwd_prep(hd, o, dout, delta=None):
    import torch
    rows = o.shape[0]
    if delta is None:
        delta = torch.empty(hd.hq, rows, dtype=torch.float32, device=o.device)
    C.bsm_bwd_prep(hd, rows, _ptr(o), _ptr(dout), _ptr(delta), _stream())
    return delta


def bwd_workspace(dp: DevicePlan, hd, device="cuda"):
    """The workspace bsm_bwd_step_ws needs for this plan (None when no step splits)."""
    import torch
    slots = dp.info["bwd_workspace_slots"]
    if slots == 0:
        return None
    return torch.empty(slots * hd.hkv * 2 * 128 * 128, dtype=torch.float32, device=device)


def bwd_step(dp: DevicePlan, s, hd, q, k, v, dout, lse, delta, dq, dk, dv, workspace=None, kv_stream=None):
    """One backward ring step against shard j = (r - s) mod R: dq carried
    (first step with work overwrites), dk/dv of shard j added to.  With a
    workspace (bwd_workspace), long dK/dV lists may be split.  With kv_stream
    (a torch stream), the dK/dV update goes there and dq's on the current
    stream (bsm_bwd_step_streams); the caller orders the inputs before both
    and joins them before reading the gradients."""
    if kv_stream is not None:
        nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        C.bsm_bwd_step_streams(dp.handle, s, hd, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                               _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), nbytes,
                               _stream(), kv_stream.cuda_stream)
    elif workspace is None:
        C.bsm_bwd_step(dp.handle, s, hd, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta),
                       _ptr(dq), _ptr(dk), _ptr(dv), _stream())
    else:
        C.bsm_bwd_step_ws(dp.handle, s, hd, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                          _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream())


# The dK/dV launches of successive steps may overlap (each writes its own
# shard's accumulators), and two of them side by side fill each other's launch
# tails.  A unit (one key tile and KV head) loops over the query tiles that
# reach it.  When some step's units average more legal queries per key than
# this, the units fill the chip for several rounds at one workgroup per CU and
# a concurrent launch of the next step takes CUs from those rounds; there one
# side stream is kept.
SHORT_UNIT_QUERIES = 4096


def kv_side_streams(dp: DevicePlan):
    """How many side streams the dK/dV launches of a backward should alternate
    between: 2 when every step's units are short (see SHORT_UNIT_QUERIES), else 1."""
    items, pairs = dp.info["bwd_items"], dp.info["step_pairs"]
    longest = max((pairs[s] / (128.0 * items[s]) for s in range(dp.ranks) if items[s] > 0), default=0.0)
    return 2 if longest <= SHORT_UNIT_QUERIES else 1


_SIDE_STREAMS = {}


def _side_streams(device, n):
    """The first n of two side streams kept per device for the forward's two
    chains and the backward's dK/dV launches.
    Streams share the device's few hardware queues; one taken afresh per call
    can land on the current stream's queue and run behind its work, so the
    same ones serve every call."""
    import torch
    idx = torch.device(device).index
    idx = torch.cuda.current_device() if idx is None else idx
    if idx not in _SIDE_STREAMS:
        _SIDE_STREAMS[idx] = [torch.cuda.Stream(device=idx) for _ in range(2)]
    return _SIDE_STREAMS[idx][:n]


def bwd_ring(dp: DevicePlan, hd, q, k_shards, v_shards, dout, o, lse, grads=None, steps=None,
             split=True, two_streams=True, kv_streams=None):
    """Backward over ring steps s = 0..R-1.  Returns (dq, dk_shards, dv_shards) in fp32.

    dk/dv shards are accumulated (+=) by the kernels: they are cleared here
    first, as the owner of a travelling accumulator would before the first
    contribution.  split: give the steps a workspace so long dK/dV lists can
    be split (bsm_bwd_step_ws).  two_streams: run every step's dK/dV update
    on a second stream beside the dQ chain (bsm_bwd_step_streams), so each
    kernel's launch tail is filled by the other's work; the gradients are
    bit-identical either way.  kv_streams (with two_streams): how many side
    streams the dK/dV launches of successive steps alternate between, each
    with its own workspace; None picks kv_side_streams(dp).  The launches of
    different steps write different shards' accumulators, so they may
    overlap."""
    import torch
    rows = dp.rows
    _need(dout, torch.bfloat16, (rows, hd.hq, hd.d), "dout")
    delta = bwd_prep(hd, o, dout)
    if grads is None:
        dq = torch.empty(rows, hd.hq, hd.d, dtype=torch.float32, device=q.device)
        dks = [torch.zeros(rows, hd.hkv, hd.d, dtype=torch.float32, device=q.device)
               for _ in range(dp.ranks)]
        dvs = [torch.zeros(rows, hd.hkv, hd.d, dtype=torch.float32, device=q.device)
               for _ in range(dp.ranks)]
    else:
        dq, dks, dvs = grads
        for t in dks + dvs:
            t.zero_()
    main = torch.cuda.current_stream()
    if two_streams:
        nside = kv_side_streams(dp) if kv_streams is None else int(kv_streams)
        if nside not in (1, 2):
            raise ValueError(f"kv_streams: expected 1 or 2, got {kv_streams}")
        sides = _side_streams(q.device, nside)
        for side in sides:
            side.wait_stream(main)  # delta and the cleared accumulators
    else:
        sides = [None]
    wss = [bwd_workspace(dp, hd, q.device) if split else None for _ in sides]
    launch = 0
    for s in (range(dp.ranks) if steps is None else steps):
        j = (dp.rank - s) % dp.ranks
        i = launch % len(sides)
        bwd_step(dp, s, hd, q, k_shards[j], v_shards[j], dout, lse, delta, dq, dks[j], dvs[j], wss[i],
                 kv_stream=sides[i])
        launch += dp.info["bwd_items"][s] > 0
    for side in sides:
        if side is not None:
            # joined before returning: whatever reuses these buffers later on
            # the current stream runs after the side streams' work
            main.wait_stream(side)
    return dq, dks, dvs
