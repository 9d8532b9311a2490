"""CPU checks of bench.py's contract pieces that need no GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True)
    assert out.returncode == 2
    assert "one GPU" in json.loads(out.stdout.strip())["error"]


def test_traffic_only_for_matching_sources():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.measured_traffic("packed_text_32k") is None
    v = bench.measured_traffic("packed_multimodal_64k")
    # either the committed summary matches the current forward sources, or it is
    # stale and reported as unknown
    assert v is None or v > 1e8


def test_planner_timing_and_algorithmic_bytes_on_cpu():
    """The host-only pieces of the bench line: planner timing at 1 and all
    threads, and the forward's algorithmic bytes (positive, one per step with
    work, state elided at a tile's first and last step)."""
    sys.path.insert(0, ROOT)
    import bench
    import numpy as np
    import block_sparse_masked_metadata_amd as bsm
    from workloads import config
    lay = config(2)
    t = bench.planner_timing(bsm, lay)
    assert t["threads_1_s"] > 0 and t["threads_all_s"] > 0 and t["cores"] >= 1
    plan = bsm.Plan.from_layout(lay)
    r, S = plan.info["busiest_rank"], plan.info["shard_tokens"]
    per = bench.fwd_algorithmic_bytes(plan, r, lay.ranks, S, lay.hq, lay.hkv, 128)
    pairs = plan.pairs()[r]
    assert len(per) == int((pairs > 0).sum()) and all(b > 0 for b in per)
    single = bench.fwd_algorithmic_bytes(plan, r, lay.ranks, S, lay.hq, lay.hkv, 128, single=True)[0]
    assert single < sum(per)  # the single pass moves no carried state


def test_backward_algorithmic_bytes_closed_form():
    """Sliding window 128K, rank 1: step 0 pairs every one of its 128 query
    tiles with all 128 key tiles of its own clip (dQ not read: first step);
    step 1 pairs query tiles 0..31 with the previous clip's last 32 key tiles
    (4095 * 4096 / 2 pairs).  Bytes per the accounting in bwd_algorithmic,
    with d = 128, Hq = 16, Hkv = 4."""
    sys.path.insert(0, ROOT)
    import bench
    import block_sparse_masked_metadata_amd as bsm
    from workloads import config
    lay = config(4)
    plan = bsm.Plan.from_layout(lay)
    w = bench.bwd_algorithmic(plan, 1, 8, 16384, 16, 4, 128)
    assert [x["step"] for x in w] == [0, 1]
    assert [x["pairs"] for x in w] == [16384 * 16384, 4095 * 4096 // 2]
    q_row = (4 * 128 + 8) * 16 + 4 * 128 * 16          # Q, dO, LSE, delta, dQ write
    assert w[0]["dq_bytes"] == 16384 * q_row + 16384 * 4 * 128 * 4
    assert w[1]["dq_bytes"] == 4096 * (q_row + 4 * 128 * 16) + 4096 * 4 * 128 * 4
    k_row = 4 * 128 * 4 + 16 * 128 * 4                   # K, V, dK and dV read + write
    assert w[0]["dkdv_bytes"] == 16384 * k_row + 16384 * (4 * 128 + 8) * 16
    assert w[1]["dkdv_bytes"] == 4096 * k_row + 4096 * (4 * 128 + 8) * 16
    line = bench.kernel_line(8 * 128 * 16 * w[0]["pairs"], w[0]["dkdv_bytes"], 10000.0, 2)
    assert line["bound"] == "mfma" and 0 < line["frac"] < 1
