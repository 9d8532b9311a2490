"""Host-side checks of libbsm (no GPU): exported symbols, the C++ planner
against the oracle planner (byte equality), error codes and determinism."""
import os
import re

import numpy as np
import pytest

import block_sparse_masked_metadata_amd as bsm
from block_sparse_masked_metadata_amd import _capi as C
from workloads import (random_small, packed_text, packed_multimodal, sliding_window,
                       long_mixed, WINDOW_INF)
from oracle import planner as oplan

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "bsm.h")


def test_exports_every_declared_symbol():
    src = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(bsm_[a-z_0-9]+)\s*\(", src, re.M))
    assert declared == set(C.EXPORTS)
    import ctypes
    lib = ctypes.CDLL(C.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert C.bsm_version() >= 100


def _compare(lay, ranks, block, order, explicit=None):
    tr = lay.tracks()
    op = oplan.build(tr, lay.window, ranks, block, order, explicit)
    p = bsm.Plan(tr, lay.window, ranks, block, order, explicit)
    assert np.array_equal(p.permutation(), op.perm.astype(np.int32))
    cost, owner = p.block_cost()
    assert np.array_equal(cost, op.cost)
    assert np.array_equal(owner, op.owner.astype(np.int32))
    pairs = p.pairs()
    for r in range(ranks):
        for s in range(ranks):
            mp, tot = p.step_map(r, s)
            omp, otot = op.step_map(r, s)
            assert np.array_equal(mp, omp), (r, s)
            assert tot == otot and pairs[r, s] == otot
    assert p.info["busiest_rank"] == op.busiest_rank()
    assert p.info["total_pairs"] == int(op.cost.sum())
    return p, op


@pytest.mark.parametrize("seed", range(24))
def test_planner_matches_oracle_tiny(seed):
    rng = np.random.default_rng(500 + seed)
    ranks = [1, 2, 3, 4, 8][seed % 5]
    block = [4, 8, 16, 128][seed % 4]
    order = ["contiguous", "ptrr"][seed % 2]
    n = block * ranks * int(rng.integers(1, 4))
    if order == "contiguous" and seed % 3 == 0:
        n += ranks
    lay = random_small(rng, n)
    _compare(lay, ranks, block, order)


def test_planner_explicit_zigzag():
    n = 64
    tr = (np.zeros(n, np.int32), -np.ones(n, np.int32), -np.ones(n, np.int32),
          np.arange(n, dtype=np.int32))
    from workloads.layouts import Layout
    lay = Layout("causal", *tr, WINDOW_INF, 4, "explicit")
    _compare(lay, 4, 8, "explicit", [0, 7, 1, 6, 2, 5, 3, 4])


@pytest.mark.parametrize("maker", [
    lambda: packed_text(),
    lambda: packed_multimodal(),
    lambda: sliding_window(n=16384, clip=2048, window=512),
    lambda: long_mixed(n=65536, clip=4096),
], ids=["packed_text_32k", "packed_multimodal_64k", "sliding_window_small", "long_mixed_small"])
def test_planner_matches_oracle_configs(maker):
    lay = maker()
    _compare(lay, lay.ranks, 128, lay.order)


@pytest.mark.slow
@pytest.mark.parametrize("maker", [sliding_window, long_mixed], ids=["sliding_window_128k", "long_mixed_1m"])
def test_planner_matches_oracle_full_size(maker):
    """The two largest layouts at full size: permutation, per-tile cost and
    owner, busiest rank, and every rank's step maps and pair counts byte-equal
    with the enumeration of the oracle planner (minutes of CPU)."""
    lay = maker()
    _compare(lay, lay.ranks, 128, lay.order)


def test_full_size_closed_forms():
    """Sliding-window 128K and long-mixed 1M layouts: pair totals against closed
    forms, and the window tile map (C++ planner only; the oracle is too slow here)."""
    lay = sliding_window()
    p = bsm.Plan.from_layout(lay)
    pairs = p.pairs()
    assert p.info["busiest_rank"] == 1
    assert int(pairs[1].sum()) == 276_822_016
    assert int(pairs.sum()) == 2_197_803_008
    mp1, _ = p.step_map(1, 1)
    want = np.zeros((128, 128), np.uint8)
    for a in range(32):
        want[a, a + 96] = C.BSM_TILE_PARTIAL
        want[a, a + 97:] = C.BSM_TILE_FULL
    assert np.array_equal(mp1, want)
    assert np.all(p.step_map(1, 0)[0] == C.BSM_TILE_FULL)
    for s in range(2, 8):
        assert not p.step_map(1, s)[0].any()
    lay = long_mixed()
    p = bsm.Plan.from_layout(lay)
    want = 0
    for a, b, mode, _ in lay.spans:
        ln = b - a
        want += ln * ln if mode == "full" else ln * (ln + 1) // 2
    assert p.info["total_pairs"] == want
    assert int(p.pairs().sum()) == want


def test_deterministic_and_thread_independent():
    lay = packed_multimodal()
    a = bsm.Plan(lay.tracks(), lay.window, 8, 128, "ptrr", threads=1)
    b = bsm.Plan(lay.tracks(), lay.window, 8, 128, "ptrr", threads=7)
    assert np.array_equal(a.permutation(), b.permutation())
    for s in range(8):
        assert np.array_equal(a.step_map(3, s)[0], b.step_map(3, s)[0])


def test_invalid_metadata_errors():
    n = 256
    good = [np.zeros(n, np.int32), -np.ones(n, np.int32), -np.ones(n, np.int32),
            np.arange(n, dtype=np.int32)]
    bad_cases = []
    s = good[0].copy(); s[10] = 5; s[11] = 1
    bad_cases.append(([s] + good[1:], WINDOW_INF, 2, "ptrr"))           # samples not contiguous
    p = good[3].copy(); p[5] = -3
    bad_cases.append((good[:3] + [p], WINDOW_INF, 2, "ptrr"))            # pos < 0
    g = good[1].copy(); g[0] = -2
    bad_cases.append(([good[0], g] + good[2:], WINDOW_INF, 2, "ptrr"))  # seg < -1
    s = good[0].copy(); s[:100] = -1
    bad_cases.append(([s] + good[1:], WINDOW_INF, 2, "ptrr"))           # negative sample id
    bad_cases.append(([s] + good[1:], WINDOW_INF, 2, "contiguous"))     # (kernels pad with -1)
    bad_cases.append((good, 0, 2, "ptrr"))                                # window < 1
    bad_cases.append((good, WINDOW_INF, 3, "ptrr"))                       # n % (128*R) != 0
    bad_cases.append((good, WINDOW_INF, 3, "contiguous"))                 # n % R != 0
    bad_cases.append((good, WINDOW_INF, 65, "contiguous"))                # too many ranks
    for tracks, w, r, order in bad_cases:
        with pytest.raises(bsm.BsmError) as e:
            bsm.Plan(tracks, w, r, 128, order)
        assert e.value.code == C.BSM_E_INVALID
        assert C.bsm_last_error()
    with pytest.raises(bsm.BsmError):
        bsm.Plan(good, WINDOW_INF, 2, 128, "explicit", [0, 0])
    # device plans need 128-token tiles
    p = bsm.Plan(good, WINDOW_INF, 2, 64, "ptrr")
    with pytest.raises(bsm.BsmError) as e:
        C.bsm_dplan_bytes(p.handle, 0)
    assert e.value.code == C.BSM_E_UNSUPPORTED


def test_single_hip_runtime_in_process():
    """libbsm must bind to the HIP runtime torch already loaded (two runtimes
    in one process crash on the first device call)."""
    import subprocess
    import sys
    code = ("import block_sparse_masked_metadata_amd, torch, re;"
            "m=open('/proc/self/maps').read();"
            "print(sorted(set(re.findall(r'\\S*libamdhip64\\S*', m))))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    libs = eval(out.stdout.strip().splitlines()[-1])
    assert len(libs) == 1, libs


def test_kv_side_streams_rule():
    """Two dK/dV side streams only when every step's key tiles average at most
    SHORT_UNIT_QUERIES legal queries per key; steps without work are ignored."""
    from types import SimpleNamespace
    from block_sparse_masked_metadata_amd.ring import SHORT_UNIT_QUERIES as T

    def dp(items, pairs):
        return SimpleNamespace(ranks=len(items), info={"bwd_items": items, "step_pairs": pairs})
    assert bsm.kv_side_streams(dp([4, 2, 0], [4 * 128 * 600, 2 * 128 * T, 0])) == 2
    assert bsm.kv_side_streams(dp([4, 2, 0], [4 * 128 * 600, 2 * 128 * T + 1, 0])) == 1
    assert bsm.kv_side_streams(dp([4, 1], [4 * 128 * 16384, 128 * 2048])) == 1
    assert bsm.kv_side_streams(dp([0, 0], [0, 0])) == 2
