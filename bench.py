#!/usr/bin/env python3
"""Benchmark: effective masked-attention TFLOP/s of one ring rank's share on one GPU.

Workload (default): the packed multimodal layout, 65536 tokens (text spans,
1024-token image pairs grouped bidirectionally, generated images with p=0.3),
24 query / 24 key-value heads, d=128, bf16, P=8 simulated ring steps on the
busiest rank's 8192-token PTRR shard.

One timed step = the whole hot path on resident inputs: P forward ring steps
(fp32 state carried in HBM, finalize on each tile's last step), the backward
prep (delta = rowsum(dO * O)), clearing the rank's own shard's dK/dV
accumulators, and P backward ring steps (dQ carried, dK/dV added into each
shard's travelling accumulator).  The planner runs once per packed batch before timing (it is reused by
every layer), as do plan upload and the input permutation.

Only unmasked FLOPs count: 4*d*Hq per legal (query, key) pair forward,
10*d*Hq backward.  `value` is the forward rate (the forward is the quoted
pass of this workload); the forward+backward rate is reported beside it.
The roofline's average launch duration comes from HIP events around each
forward launch of the last timed pass.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import platform
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, 2.4 GHz (AMD spec)
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3,
                    help="workload index 1..5; 6 = video frames in one group per sample (layout transforms)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU seconds of the oracle baseline sample")
    ap.add_argument("--fwd-only", action="store_true", help="time only the forward pass")
    ap.add_argument("--single", action="store_true",
                    help="diagnostic: time the one-launch single pass instead of the ring steps")
    ap.add_argument("--merge", choices=["carry", "fp32", "bf16"], default="carry",
                    help="accuracy controls: time per-step merges instead of the fp32 carry "
                         "(forward only; no roofline)")
    ap.add_argument("--fetch", action="store_true",
                    help="sparse fetch: contiguous chunks, one pass over the rank's shard and its "
                         "fetched remote tiles (forward only; the fetch itself is not timed)")
    ap.add_argument("--order", choices=["ptrr", "contiguous"], default=None,
                    help="token order of the ring layout (default: the workload's own)")
    ap.add_argument("--vision-group", action="store_true",
                    help="permute tokens into the vision-group order before planning (layout transform)")
    ap.add_argument("--chunks", type=int, default=0,
                    help="chunked ring layout: search 1..K contiguous chunks per rank")
    ap.add_argument("--tau", type=float, default=0.0,
                    help="chunk search: cost of one extra key range per rank and step, in pairs")
    ap.add_argument("--dense", action="store_true",
                    help="dense-call mode: every ring step as full / causal / reverse calls")
    ap.add_argument("--ring-estimate", action="store_true",
                    help="also time every rank's forward steps and report the ring's critical "
                         "path (sum over steps of the slowest rank), untimed by the headline")
    ap.add_argument("--fit-tau", action="store_true",
                    help="fit the chunk cost's per-range term: time the ring critical path at "
                         "1, 2, 4, ..., 64 chunks per rank and print one JSON line with the fit")
    ap.add_argument("--fwd-chains", type=int, choices=(1, 2), default=None,
                    help="forward ring: 1 launch per step, or the plan's two chains of query tiles on "
                         "two streams (default: as fwd_chains picks for the plan)")
    ap.add_argument("--kv-streams", type=int, choices=(1, 2), default=None,
                    help="backward: side streams the dK/dV launches alternate over "
                         "(default: as kv_side_streams picks for the plan)")
    ap.add_argument("--one-stream", action="store_true",
                    help="backward: the dK/dV launches on the same stream as the dQ launches "
                         "(counter runs; no per-kernel backward roofline)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    return ap.parse_args()


HERE = os.path.dirname(os.path.abspath(__file__))
FWD_SOURCES = ["block_sparse_masked_metadata_amd/csrc/fwd.hip",
               "block_sparse_masked_metadata_amd/csrc/kernels.hpp",
               "block_sparse_masked_metadata_amd/csrc/tile_common.hpp",
               "block_sparse_masked_metadata_amd/csrc/capi.hip"]  # the packer sets the item order
TRAFFIC_PROFILE = "profiles/fwd_kernel_hbm_packed_multimodal_64k.md"


def measured_traffic(workload):
    """HBM bytes per forward launch from the committed counter summary, or None
    when it is for another workload or the kernel sources changed since."""
    import hashlib
    if workload != "packed_multimodal_64k":
        return None
    try:
        text = open(os.path.join(HERE, TRAFFIC_PROFILE)).read()
        h = hashlib.sha256()
        for f in FWD_SOURCES:
            h.update(open(os.path.join(HERE, f), "rb").read())
        kv = dict(line.split(" = ", 1) for line in text.splitlines() if " = " in line)
        if kv.get("sources_sha256", "").strip() != h.hexdigest():
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def fwd_algorithmic_bytes(plan, r, R, S, hq, hkv, d, single=False):
    """HBM bytes the forward must move, per launch, from the plan's tile maps.

    Per ring step s: Q of the query tiles with work (2*d*Hq per row); K and V of
    the key tiles that appear in any of their lists (4*d*Hkv per key); the fp32
    state (O_acc, m, l: (4*d + 8)*Hq per row) read unless it is the tile's first
    step with work and written unless it is its last; at the last step O (bf16)
    and LSE instead (2*d + 4 bytes per row and head).  The single pass moves Q,
    the needed key tiles of every shard and the final O/LSE once."""
    T = plan.info["tiles_per_shard"]
    rows = np.minimum(128, S - 128 * np.arange(T)).astype(np.int64)
    active, keyset = [], []
    for s in range(R):
        mp, _ = plan.step_map(r, s)
        active.append((mp > 0).any(axis=1))
        keyset.append((mp > 0).any(axis=0))
    act = np.array(active)                      # [R, T]
    has = act.any(axis=0)
    first = np.where(has, act.argmax(axis=0), -1)
    last = np.where(has, R - 1 - act[::-1].argmax(axis=0), -1)
    state_row = (4 * d + 8) * hq
    if single:
        qrows = int(rows[has].sum())
        kv = sum(int(rows[keyset[s]].sum()) for s in range(R)) * 4 * d * hkv
        return [qrows * 2 * d * hq + kv + qrows * (2 * d + 4) * hq]
    out = []
    for s in range(R):
        a = act[s]
        if not a.any():
            continue
        q = int(rows[a].sum()) * 2 * d * hq
        kv = int(rows[keyset[s]].sum()) * 4 * d * hkv
        rd = int(rows[a & (first != s)].sum()) * state_row
        wr = int(rows[a & (last != s)].sum()) * state_row
        fin = int(rows[a & (last == s)].sum()) * (2 * d + 4) * hq
        out.append(q + kv + rd + wr + fin)
    return out


def bwd_algorithmic(plan, r, R, S, hq, hkv, d):
    """Per backward step with work: legal pairs and the HBM bytes each kernel
    must move, from the plan's tile maps.

    bwd_dq (per query tile with work): Q and dO (4*d*Hq per row), LSE and
    delta (8*Hq), the fp32 dQ written (4*d*Hq) and read unless it is the tile's
    first step with work, and K and V of the key tiles in its lists (4*d*Hkv
    per key).  bwd_dkdv (per key tile with work): K and V (4*d*Hkv per key),
    the shard's fp32 dK and dV read and written (16*d*Hkv per key), and Q, dO,
    LSE and delta of the query tiles in its lists ((4*d + 8)*Hq per row)."""
    T = plan.info["tiles_per_shard"]
    rows = np.minimum(128, S - 128 * np.arange(T)).astype(np.int64)
    maps = [plan.step_map(r, s) for s in range(R)]
    act = np.array([(mp > 0).any(axis=1) for mp, _ in maps])   # [R, T] query tiles with work
    has = act.any(axis=0)
    first = np.where(has, act.argmax(axis=0), -1)
    out = []
    for s in range(R):
        mp, pairs = maps[s]
        qa = act[s]
        if not qa.any():
            continue
        ka = (mp > 0).any(axis=0)                               # key tiles with work
        qrows, krows = int(rows[qa].sum()), int(rows[ka].sum())
        dq = qrows * ((4 * d + 8) * hq + 4 * d * hq) + int(rows[qa & (first != s)].sum()) * 4 * d * hq \
            + krows * 4 * d * hkv
        dkdv = krows * (4 * d * hkv + 16 * d * hkv) + qrows * (4 * d + 8) * hq
        out.append({"step": s, "pairs": int(pairs), "dq_bytes": dq, "dkdv_bytes": dkdv})
    return out


def kernel_line(flops, nbytes, us, launches, credited=None):
    """Roofline of one kernel from its per-launch algorithmic work and its
    average launch duration: bound by the longer of the MFMA and HBM times."""
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    tf = flops / (us * 1e-6) / 1e12
    gbs = nbytes / (us * 1e-6) / 1e9
    if t_hbm > t_mfma:
        bound, achieved, peak, unit = "hbm", gbs, PEAK_HBM_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s"
    line = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "algorithmic_bytes": int(nbytes),
            "executed_flops": int(flops), "avg_launch_us": round(us, 2), "launches_per_step": launches,
            "mfma_tflops": round(tf, 2), "hbm_gbs": round(gbs, 1)}
    if credited is not None:
        line["credited_flops"] = int(credited)
    return line


def pass_rates(bsm, torch, hd, S, hq, d, reps=20):
    """HBM rate of the elementwise passes on the share's shape (untimed by the
    headline): the two accuracy-control merges of a ring step, with every row
    reached.  Algorithmic bytes: merge_bf16 reads O_run, O_s (bf16) and both
    LSEs and writes O_run and LSE_run: (6*d + 12)*Hq per row; merge_fp32 reads
    O_run (fp32), the step's O_acc, m, l and LSE_run and writes O_run and
    LSE_run: (12*d + 16)*Hq per row."""
    C = bsm._capi
    st = torch.cuda.current_stream().cuda_stream
    g = torch.Generator(device="cuda").manual_seed(1)
    o_run = torch.randn(S, hq, d, device="cuda", generator=g).to(torch.bfloat16)
    o_s = torch.randn(S, hq, d, device="cuda", generator=g).to(torch.bfloat16)
    lse_run = torch.zeros(hq, S, device="cuda")
    lse_s = torch.zeros(hq, S, device="cuda")
    acc, m, l = bsm.new_state(S, hq, d)
    acc.normal_(generator=g)
    m.zero_()
    l.fill_(1.0)
    o32 = torch.randn(S, hq, d, device="cuda", generator=g)
    calls = {
        "merge_bf16": ((6 * d + 12) * hq * S, lambda: C.bsm_fwd_merge_bf16(
            hd, S, o_run.data_ptr(), lse_run.data_ptr(), o_s.data_ptr(), lse_s.data_ptr(), st)),
        "merge_fp32": ((12 * d + 16) * hq * S, lambda: C.bsm_fwd_merge_fp32(
            hd, S, o32.data_ptr(), lse_run.data_ptr(), acc.data_ptr(), m.data_ptr(), l.data_ptr(), None, st)),
    }
    out = {}
    for name, (nbytes, fn) in calls.items():
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out[name] = {"algorithmic_bytes": int(nbytes), "avg_launch_us": round(us, 2),
                     "hbm_gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    return out


def sparse_fetch_summary(lay, plan, r):
    """Remote key tiles the measured rank needs under this plan's order and
    under contiguous chunks (MARBLE section 04: the sparse all-to-all moves only
    those; the ring moves all R - 1 remote shards)."""
    import dataclasses
    import block_sparse_masked_metadata_amd as bsm
    R, T = plan.info["ranks"], plan.info["tiles_per_shard"]
    out = {"remote_tiles": (R - 1) * T}
    _, out[f"needed_{lay.order}"] = plan.fetch_set(r)
    if lay.order != "contiguous":
        cp = bsm.Plan.from_layout(dataclasses.replace(lay, order="contiguous"))
        _, out["needed_contiguous"] = cp.fetch_set(cp.info["busiest_rank"])
    out["bytes_avoided_contiguous"] = round(1 - out["needed_contiguous"] / out["remote_tiles"], 4) \
        if out["remote_tiles"] else 0.0
    return out


def cpu_baseline(lay, plan_pairs_fn, rows_all, q, k, v, target_s):
    """Time the fp64 oracle on whole samples of the measured rank's share."""
    from oracle import attention as oatt
    from oracle.mask import legal, take
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    sample = lay.sample
    ranges = oatt.sample_ranges(sample)
    smp_of_row = sample[rows_all]
    order = list(dict.fromkeys(smp_of_row.tolist()))
    rng = np.random.default_rng(0)
    rng.shuffle(order)
    done_rows, pairs, used = 0, 0, []
    t0 = time.perf_counter()
    for sid in order:
        sel = rows_all[smp_of_row == sid]
        a, b = ranges[sid]
        pairs += int(legal(take(lay.tracks(), sel), take(lay.tracks(), np.arange(a, b)),
                           lay.window).sum())
        oatt.forward_rows(lay.tracks(), lay.window, q, k, v, sel, 1.0 / np.sqrt(lay.d))
        done_rows += len(sel)
        used.append(sid)
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    flops = 4 * lay.d * lay.hq * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 oracle forward of {done_rows} query rows of the measured rank "
                      f"({len(used)} whole samples, {pairs} legal pairs) in {dt:.1f} s; "
                      f"host {platform.processor() or platform.machine()}, "
                      f"{len(os.sched_getaffinity(0))} cores in the affinity mask"}


def mfma_probe(torch):
    """Dense bf16 MFMA rate and shader clock measured on this GPU with the
    probe library (independent MFMA chains on every SIMD); None if it is not
    built."""
    import ctypes
    path = os.path.join(HERE, "block_sparse_masked_metadata_amd", "libbsm_probe.so")
    if not os.path.exists(path):
        return None
    fn = ctypes.CDLL(path).bsm_probe_mfma
    fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * cus, 4000  # two workgroups per CU: two waves per SIMD
    stamps = torch.zeros(blocks * 16, dtype=torch.int64, device="cuda")
    sink = torch.zeros(blocks * 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    assert fn(blocks, 200, stamps.data_ptr(), sink.data_ptr(), stream) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    assert fn(blocks, iters, stamps.data_ptr(), sink.data_ptr(), stream) == 0
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    st = stamps.view(-1, 4).cpu().double()
    clock = float(((st[:, 1] - st[:, 0]) / (st[:, 3] - st[:, 2])).median()) * 0.1  # real-time counter: 100 MHz
    return {"tflops": round(blocks * 4 * iters * 8 * 32768 / (ms * 1e-3) / 1e12, 1),
            "clock_ghz": round(clock, 3), "cus": cus,
            "kind": "v_mfma_f32_32x32x16_bf16, 8 independent chains per wave, 2 waves per SIMD"}


def planner_timing(bsm, lay):
    """Host planner wall time at one thread and at every core of this process."""
    cores = len(os.sched_getaffinity(0))
    out = {}
    for name, th in (("threads_1_s", 1), ("threads_all_s", cores)):
        t0 = time.perf_counter()
        bsm.Plan.from_layout(lay, threads=th)
        out[name] = round(time.perf_counter() - t0, 4)
    out["cores"] = cores
    return out


def ring_estimate(bsm, torch, plan, hd, full, perm, k_all, v_all, lay, d, passes, dense=False):
    """Every rank's forward steps on this one GPU, each launch timed with
    events: the ring's forward critical path is the sum over steps of the
    slowest rank's launch (communication and overlap not included)."""
    R, S = lay.ranks, plan.info["shard_tokens"]
    ks = [k_all[j * S:(j + 1) * S] for j in range(R)]
    vs = [v_all[j * S:(j + 1) * S] for j in range(R)]
    t = np.zeros((R, R))
    for rr in range(R):
        dpr = bsm.DevicePlan(plan, rr, dense=dense)
        q = full[0][torch.from_numpy(perm[rr * S:(rr + 1) * S]).cuda()].contiguous()
        state = bsm.new_state(S, lay.hq, d)
        o = torch.empty(S, lay.hq, d, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(lay.hq, S, dtype=torch.float32, device="cuda")
        steps = [s for s in range(R) if dpr.info["fwd_items"][s] > 0]
        for it in range(passes + 1):
            ev = []
            for s in steps:
                j = (rr - s) % R
                ev.append(torch.cuda.Event(enable_timing=True))
                ev[-1].record()
                bsm.fwd_step(dpr, s, hd, q, ks[j], vs[j], state, o, lse)
                ev.append(torch.cuda.Event(enable_timing=True))
                ev[-1].record()
            torch.cuda.synchronize()
            if it:  # the first pass warms up
                for i, s in enumerate(steps):
                    t[rr, s] += ev[2 * i].elapsed_time(ev[2 * i + 1]) / passes
        del dpr, q, state, o, lse
    pairs = plan.pairs()
    return {"critical_path_ms": round(float(t.max(axis=0).sum()), 4),
            "busiest_rank_ms": round(float(t.sum(axis=1).max()), 4),
            "mean_rank_ms": round(float(t.sum(axis=1).mean()), 4),
            "step_max_pairs_sum": int(pairs.max(axis=0).sum()),
            "busiest_rank_pairs": int(pairs.sum(axis=1).max()),
            "passes": passes}


def fit_tau(args, bsm, torch, lay, config_qkv):
    """Chunk cost C = sum_s max_r W[r][(r - s) mod R] + tau * R * k: least squares
    of the measured forward critical path t_k = a * P_k + c * R * k + b over chunk
    counts k (P_k the planner's step-max sum), tau = c / a in pairs."""
    import dataclasses
    d = 128
    hd = bsm.heads(lay.hq, lay.hkv, d, 1.0 / np.sqrt(lay.d))
    full = config_qkv(lay.n, lay.hq, lay.hkv, d, lay.seed, "cuda")
    base = bsm.Plan.from_layout(dataclasses.replace(lay, order="contiguous"))
    R = lay.ranks
    rows = []
    for k in (1, 2, 4, 8, 16, 32, 64):
        try:
            bperm, ci = base.chunk_order(k, k, 0.0, 4)
        except bsm.BsmError:
            break  # fewer blocks than chunks
        chl = dataclasses.replace(lay, order="explicit", block_perm=bperm)
        plan = bsm.Plan.from_layout(chl)
        perm = plan.permutation().astype(np.int64)
        pidx = torch.from_numpy(perm).cuda()
        k_all = full[1][pidx].contiguous()
        v_all = full[2][pidx].contiguous()
        est = ring_estimate(bsm, torch, plan, hd, full, perm, k_all, v_all, lay, d,
                            max(1, args.steps // 4), args.dense)
        rows.append({"k": k, "strategy": ci["strategy"], "step_max_pairs": int(ci["step_max_sum"]),
                     "critical_path_ms": est["critical_path_ms"]})
        del k_all, v_all
    P = np.array([r_["step_max_pairs"] for r_ in rows], float)
    K = np.array([R * r_["k"] for r_ in rows], float)
    t = np.array([r_["critical_path_ms"] for r_ in rows], float)
    A = np.stack([P, K, np.ones_like(P)], axis=1)
    (a, c, b), *_ = np.linalg.lstsq(A, t, rcond=None)
    pred = A @ np.array([a, c, b])
    for r_, p_ in zip(rows, pred):
        r_["predicted_ms"] = round(float(p_), 4)
    return {"metric": "chunk cost fit", "workload": lay.name, "mode": "dense calls" if args.dense else "block-sparse",
            "ranks": R, "ms_per_pair": float(a), "ms_per_range": float(c), "ms_fixed": float(b),
            "tau_pairs": float(c / a) if a > 0 else None,
            "max_rel_err": round(float(np.max(np.abs(pred - t) / t)), 4), "points": rows}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; --gpus must be 1"}))
        sys.exit(2)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import torch
    import block_sparse_masked_metadata_amd as bsm
    from workloads import config, qkv

    import dataclasses
    lay = config(args.config)
    if args.fit_tau:
        print(json.dumps(fit_tau(args, bsm, torch, lay, qkv)), flush=True)
        return
    if args.vision_group:
        from workloads import permuted
        lay = permuted(lay, bsm.vision_group_order(lay.tracks()), name=lay.name + "_vision_group")
    if args.order:
        lay = dataclasses.replace(lay, order=args.order)
    if args.fetch:
        lay = dataclasses.replace(lay, order="contiguous")
    chunk_info = None
    t0 = time.perf_counter()
    if args.chunks:
        base = bsm.Plan.from_layout(dataclasses.replace(lay, order="contiguous"))
        bperm, chunk_info = base.chunk_order(1, args.chunks, args.tau, 4)
        lay = dataclasses.replace(lay, order="explicit", block_perm=bperm)
    plan = bsm.Plan.from_layout(lay)
    plan_s = time.perf_counter() - t0
    r = plan.info["busiest_rank"]
    R, S = lay.ranks, plan.info["shard_tokens"]
    dp = bsm.DevicePlan(plan, r, dense=args.dense)
    perm = plan.permutation().astype(np.int64)
    rows = perm[r * S:(r + 1) * S]
    pairs = plan.pairs()[r]
    total_pairs = int(pairs.sum())
    d = 128
    hd = bsm.heads(lay.hq, lay.hkv, d, 1.0 / np.sqrt(lay.d))
    full = qkv(lay.n, lay.hq, lay.hkv, d, lay.seed, "cuda", with_do=True)
    pidx = torch.from_numpy(perm).cuda()
    ridx = torch.from_numpy(rows).cuda()
    q = full[0][ridx].contiguous()
    dout = full[3][ridx].contiguous()
    k_all = full[1][pidx].contiguous()
    v_all = full[2][pidx].contiguous()
    ks = [k_all[j * S:(j + 1) * S] for j in range(R)]
    vs = [v_all[j * S:(j + 1) * S] for j in range(R)]
    state = bsm.new_state(S, lay.hq, d)
    o = torch.empty(S, lay.hq, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(lay.hq, S, dtype=torch.float32, device="cuda")
    dq = torch.empty(S, lay.hq, d, dtype=torch.float32, device="cuda")
    dks = [torch.zeros(S, lay.hkv, d, dtype=torch.float32, device="cuda") for _ in range(R)]
    dvs = [torch.zeros(S, lay.hkv, d, dtype=torch.float32, device="cuda") for _ in range(R)]
    fwd_steps = [s for s in range(R) if dp.info["fwd_items"][s] > 0]
    do_bwd = not args.fwd_only and args.merge == "carry" and not args.fetch
    if args.dense and args.fetch:
        print(json.dumps({"error": "--dense and --fetch exclude each other"}))
        sys.exit(2)

    if args.fetch:
        kf, vf = bsm.gather_fetched(plan, r, k_all, v_all)
    ring_mode = not (args.fetch or args.single or args.merge != "carry")

    def chain_items(s, c):
        n, c0 = dp.info["fwd_items"][s], dp.info["fwd_chain0_items"][s]
        return c0 if c == 0 else n - c0
    nchains = (args.fwd_chains or bsm.fwd_chains(dp, hd)) if ring_mode else 1
    # two side streams, made once: the forward's two chains and the
    # backward's dK/dV launches run on them (as fwd_ring and bwd_ring do).
    # Streams map onto a few hardware queues; more streams than queues would
    # put a side stream on the current stream's queue, behind its work.
    side_streams = [torch.cuda.Stream() for _ in range(2)]
    fwd_sides = side_streams if nchains == 2 else []

    def forward(events=None):
        if args.fetch:
            if events is not None:
                events.append(torch.cuda.Event(enable_timing=True))
                events[-1].record()
            bsm.fwd_fetched(dp, hd, q, kf, vf, out=(o, lse))
            if events is not None:
                events.append(torch.cuda.Event(enable_timing=True))
                events[-1].record()
            return
        if args.merge != "carry":
            if events is not None:
                events.append(torch.cuda.Event(enable_timing=True))
                events[-1].record()
            bsm.fwd_ring_merged(dp, hd, q, ks, vs, args.merge)
            if events is not None:
                events.append(torch.cuda.Event(enable_timing=True))
                events[-1].record()
            return
        if args.single:
            if events is not None:
                events.append(torch.cuda.Event(enable_timing=True))
                events[-1].record()
            bsm.fwd_single(dp, hd, q, k_all, v_all, out=(o, lse))
            if events is not None:
                events.append(torch.cuda.Event(enable_timing=True))
                events[-1].record()
            return
        if nchains == 2:
            # the plan's two chains of query tiles, each on its own stream
            # with its steps in order, as fwd_ring runs them; events (per
            # launch) on the stream the launch runs on
            main = torch.cuda.current_stream()
            for side in fwd_sides:
                side.wait_stream(main)
            for s in fwd_steps:
                j = (r - s) % R
                for c, side in enumerate(fwd_sides):
                    if chain_items(s, c) == 0:
                        continue
                    with torch.cuda.stream(side):
                        if events is not None:
                            events.append(torch.cuda.Event(enable_timing=True))
                            events[-1].record()
                        bsm.fwd_step(dp, s, hd, q, ks[j], vs[j], state, o, lse, chain=c)
                        if events is not None:
                            events.append(torch.cuda.Event(enable_timing=True))
                            events[-1].record()
            for side in fwd_sides:
                main.wait_stream(side)
            return
        for s in fwd_steps:
            j = (r - s) % R
            if events is not None:
                events.append(torch.cuda.Event(enable_timing=True))
                events[-1].record()
            bsm.fwd_step(dp, s, hd, q, ks[j], vs[j], state, o, lse)
            if events is not None:
                events.append(torch.cuda.Event(enable_timing=True))
                events[-1].record()

    delta = torch.empty(lay.hq, S, dtype=torch.float32, device="cuda")
    bwd_work = bwd_algorithmic(plan, r, R, S, lay.hq, lay.hkv, d)
    bwd_steps = {w["step"] for w in bwd_work}
    # the dK/dV launches alternate between as many side streams as bwd_ring
    # would use for this plan, each with its own workspace (which lets long
    # dK/dV lists split over the GPU)
    sides = side_streams[:args.kv_streams or bsm.kv_side_streams(dp)]
    bwss = [bsm.bwd_workspace(dp, hd) for _ in sides]

    def event(stream=None):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def backward(events=None):
        # One rank's backward: delta, then the R steps.  Shard j's dK/dV
        # accumulator travels the ring and arrives holding the other ranks'
        # contributions; only the rank's own shard (j = r) starts from zero
        # here, so the others keep accumulating across timed passes (their
        # values are not checked; the kernels do the same work either way).
        # events: per-launch events of the prep and of every step, each on
        # the stream its kernels run on (the dQ launch alone on the current
        # stream, the dK/dV launch (and its split reduction) alone on its
        # side stream).
        main = torch.cuda.current_stream()
        if events is not None:
            events["prep"].append(event())
        bsm.bwd_prep(hd, o, dout, delta)
        if events is not None:
            events["prep"].append(event())
        dks[r].zero_()
        dvs[r].zero_()
        # dQ chain on the current stream, the dK/dV launches of successive
        # steps with work alternating over the side streams, joined at the
        # end, as bwd_ring runs them by default
        for side in sides:
            side.wait_stream(main)
        launch = 0
        for s in range(R):
            j = (r - s) % R
            side, ws = sides[launch % len(sides)], bwss[launch % len(sides)]
            if events is not None and s in bwd_steps:
                events["dq"].append(event())
                events["dkdv"].append(event(side))
            bsm.bwd_step(dp, s, hd, q, ks[j], vs[j], dout, lse, delta, dq, dks[j], dvs[j], ws,
                         kv_stream=None if args.one_stream else side)
            if events is not None and s in bwd_steps:
                events["dq"].append(event())
                events["dkdv"].append(event(side))
            launch += s in bwd_steps
        for side in sides:
            main.wait_stream(side)

    # The GPU events time the gaps between markers, so a host pause between a
    # marker and the launches after it counts as GPU time: collect Python
    # garbage now and keep the collector off until the timed passes end.
    gc.collect()
    gc.disable()
    for _ in range(args.warmup):
        forward()
        if do_bwd:
            backward()
    torch.cuda.synchronize()

    launch_ev = []
    bwd_ev = {"prep": [], "dq": [], "dkdv": []}
    marks = []
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        f0 = torch.cuda.Event(enable_timing=True)
        f1 = torch.cuda.Event(enable_timing=True)
        f0.record()
        # per-launch events on the last timed pass only: recorded between
        # back-to-back launches they stretch the forward by 5-13%
        forward(launch_ev if _ == args.steps - 1 else None)
        f1.record()
        marks.append((f0, f1))
        if do_bwd:
            backward(bwd_ev if _ == args.steps - 1 and not args.one_stream else None)
    end = torch.cuda.Event(enable_timing=True)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gc.enable()

    total_ms = start.elapsed_time(end)
    fwd_each = sorted(a.elapsed_time(b) for a, b in marks)
    fwd_ms = sum(fwd_each) / args.steps
    step_ms = total_ms / args.steps
    bwd_ms = step_ms - fwd_ms if do_bwd else 0.0
    launches = [launch_ev[i].elapsed_time(launch_ev[i + 1]) for i in range(0, len(launch_ev), 2)]
    avg_launch_ms = sum(launches) / len(launches)
    fwd_flops = 4 * d * lay.hq * total_pairs
    bwd_flops = 10 * d * lay.hq * total_pairs
    fwd_tflops = fwd_flops / (fwd_ms * 1e-3) / 1e12
    nlaunch = (1 if not ring_mode else len(fwd_steps) if nchains == 1 else
               sum(chain_items(s, c) > 0 for s in fwd_steps for c in (0, 1)))
    per_launch_flops = fwd_flops / nlaunch
    per_launch_bytes = sum(fwd_algorithmic_bytes(plan, r, R, S, lay.hq, lay.hkv, d,
                                                 args.single or args.fetch)) / nlaunch
    # roofline of the forward kernel: whichever of the MFMA and HBM times of its
    # algorithmic work is longer bounds it
    t_mfma = per_launch_flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = per_launch_bytes / (PEAK_HBM_GBS * 1e9)
    mfma_tflops = per_launch_flops / (avg_launch_ms * 1e-3) / 1e12
    hbm_gbs = per_launch_bytes / (avg_launch_ms * 1e-3) / 1e9
    if t_hbm > t_mfma:
        bound, achieved, peak, unit = "hbm", hbm_gbs, PEAK_HBM_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", mfma_tflops, PEAK_BF16_TFLOPS, "TFLOP/s"

    bwd_roof = None
    if do_bwd and not args.one_stream:
        def avg_us(ev):
            return 1e3 * sum(ev[i].elapsed_time(ev[i + 1]) for i in range(0, len(ev), 2)) / (len(ev) // 2)
        nb = len(bwd_work)
        bpairs = sum(w["pairs"] for w in bwd_work)
        prep_bytes = S * lay.hq * (4 * d + 4)
        prep_us = avg_us(bwd_ev["prep"])
        bwd_roof = {
            # executed FLOPs: the dQ kernel recomputes S and dP and forms dQ
            # (6*d*Hq per pair), the dK/dV kernel recomputes S and dP and forms
            # dV and dK (8*d*Hq); the metric credits 10*d*Hq for both
            "bwd_dkdv": kernel_line(8 * d * lay.hq * bpairs / nb, sum(w["dkdv_bytes"] for w in bwd_work) / nb,
                                    avg_us(bwd_ev["dkdv"]), nb),
            "bwd_dq": kernel_line(6 * d * lay.hq * bpairs / nb, sum(w["dq_bytes"] for w in bwd_work) / nb,
                                  avg_us(bwd_ev["dq"]), nb),
            "bwd_prep": {"bound": "hbm", "algorithmic_bytes": prep_bytes, "avg_launch_us": round(prep_us, 2),
                         "hbm_gbs": round(prep_bytes / (prep_us * 1e-6) / 1e9, 1),
                         "frac": round(prep_bytes / (prep_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
            "credited_flops_per_step": int(bwd_flops),
            "executed_flops_per_step": int(14 * d * lay.hq * bpairs),
            "streams": (f"dQ launches on one stream, dK/dV launches on {len(sides)} side stream(s) "
                        "(successive steps alternating); each duration is measured on its own stream"),
        }

    if args.copy_mib:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    out = {
        "metric": "effective masked-attention TFLOP/s (fwd, fwd+bwd) and % of bf16 MFMA peak, 1 GPU",
        "value": round(fwd_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": lay.name, "tokens": lay.n, "ring_steps": R, "rank": r,
                   "query_rows": S, "hq": lay.hq, "hkv": lay.hkv, "d": d,
                   "legal_pairs": total_pairs, "layout": lay.order},
        "pct_of_peak": round(100 * fwd_tflops / PEAK_BF16_TFLOPS, 2),
        "fwd_ms": round(fwd_ms, 4),
        "fwd_ms_median_min_max": [round(float(np.median(fwd_each)), 4), round(fwd_each[0], 4),
                                  round(fwd_each[-1], 4)],
        "fwd_tflops": round(fwd_tflops, 2),
        "fwd_bwd": None if not do_bwd else {
            "ms": round(step_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "tflops": round((fwd_flops + bwd_flops) / (step_ms * 1e-3) / 1e12, 2),
            "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2),
            "pct_of_peak": round(100 * (fwd_flops + bwd_flops) / (step_ms * 1e-3) / 1e12
                                 / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"bound": bound, "kernel": "fwd_kernel", "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4),
                     "traffic": None if args.single or args.dense else measured_traffic(lay.name),
                     "algorithmic_bytes": int(per_launch_bytes),
                     "algorithmic_flops": int(per_launch_flops),
                     "flop_per_byte": round(per_launch_flops / per_launch_bytes, 1),
                     "ridge_flop_per_byte": round(PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9), 1),
                     "mfma_tflops": round(mfma_tflops, 2),
                     "mfma_frac": round(mfma_tflops / PEAK_BF16_TFLOPS, 4),
                     "hbm_gbs": round(hbm_gbs, 1),
                     "hbm_frac": round(hbm_gbs / PEAK_HBM_GBS, 4),
                     "avg_launch_us": round(avg_launch_ms * 1e3, 2),
                     "launches_per_step": nlaunch,
                     "chains": nchains,
                     "launches": ("one per ring step" if nchains == 1 else
                                  "one per ring step and chain of query tiles; the two chains run on two "
                                  "streams side by side, so each launch's duration is measured while the "
                                  "other chain's launch shares the GPU"),
                     # the whole forward's rate: every launch's algorithmic bytes over the forward's time
                     "aggregate_hbm_gbs": round(per_launch_bytes * nlaunch / (fwd_ms * 1e-3) / 1e9, 1),
                     "aggregate_hbm_frac": round(per_launch_bytes * nlaunch / (fwd_ms * 1e-3) / 1e9
                                                 / PEAK_HBM_GBS, 4)},
        "mode": ("dense calls" + (" (single pass)" if args.single else "") if args.dense else
                 "single-pass diagnostic" if args.single else
                 "sparse fetch: one pass over the shard and fetched tiles (contiguous chunks)" if args.fetch else
                 "ring" if args.merge == "carry" else f"ring, per-step {args.merge} merge (accuracy control)"),
        "sparse_fetch": sparse_fetch_summary(lay, plan, r),
        "planner_s": round(plan_s, 4),
        "wall_s": round(wall, 3),
    }
    if bwd_roof is not None:
        out["bwd_roofline"] = bwd_roof
    if args.merge != "carry":
        out["roofline"] = None  # the timed forward includes fills and merge kernels
    out["passes"] = pass_rates(bsm, torch, hd, S, lay.hq, d)
    probe = mfma_probe(torch)
    if probe:
        probe["fwd_frac"] = round(mfma_tflops / probe["tflops"], 4)  # the forward kernel, per launch
        out["mfma_probe"] = probe
    out["planner"] = planner_timing(bsm, lay)
    if chunk_info is not None:
        out["chunking"] = chunk_info
    if args.ring_estimate:
        out["ring_estimate"] = ring_estimate(bsm, torch, plan, hd, full, perm, k_all, v_all,
                                             lay, d, max(1, args.steps // 4), args.dense)
    if not args.no_cpu_baseline:
        qc, kc, vc = (t.cpu() for t in full[:3])
        out["cpu_baseline"] = cpu_baseline(lay, None, rows, qc, kc, vc, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
