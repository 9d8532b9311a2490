"""The threaded host planner under AddressSanitizer + UndefinedBehaviorSanitizer
and under ThreadSanitizer (CPU only): tests/sanitize/planner_driver.cpp builds
the plans of several layouts with 8 threads and walks every planner entry
point; the sanitizers abort on any finding."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from workloads import random_small, packed_multimodal, packed_text, video_group, permuted

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_masked_metadata_amd", "csrc")
ORDERS = {"contiguous": 0, "ptrr": 1}


def _write(path, lay):
    with open(path, "wb") as f:
        f.write(np.int64(lay.n).tobytes())
        f.write(np.array([min(lay.window, 0x7FFFFFFF), lay.ranks, ORDERS[lay.order]], np.int32).tobytes())
        for t in lay.tracks():
            f.write(np.ascontiguousarray(t, np.int32).tobytes())


def _layouts():
    rng = np.random.default_rng(77)
    out = [packed_multimodal(n=16384, ranks=4), packed_text(n=16384)]
    v = video_group(n=32768, frame=64, stamp=4, min_frames=4, max_frames=24)
    out.append(permuted(v, _vision(v)))
    for i in range(4):
        lay = random_small(rng, 128 * 4 * 3, max_span=200)
        lay.ranks, lay.order = 4, ["ptrr", "contiguous"][i % 2]
        out.append(lay if i < 2 else permuted(lay, _vision(lay)))
    return out


def _vision(lay):
    import block_sparse_masked_metadata_amd as bsm
    return bsm.vision_group_order(lay.tracks())


@pytest.mark.slow
@pytest.mark.parametrize("kind", ["address,undefined", "thread"])
def test_planner_under_sanitizer(tmp_path, kind):
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    exe = tmp_path / "driver"
    srcs = [os.path.join(ROOT, "tests", "sanitize", "planner_driver.cpp"),
            os.path.join(CSRC, "planner.cpp"), os.path.join(CSRC, "calls.cpp")]
    flags = ["-O1", "-g", "-std=c++17", "-pthread", "-fno-omit-frame-pointer", f"-fsanitize={kind}",
             "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    subprocess.run(["g++", *flags, *srcs, "-o", str(exe)], check=True, timeout=600)
    files = []
    for i, lay in enumerate(_layouts()):
        f = tmp_path / f"layout{i}.bin"
        _write(f, lay)
        files.append(str(f))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", TSAN_OPTIONS="halt_on_error=1")
    out = subprocess.run([str(exe), *files], capture_output=True, text=True, timeout=900, env=env)
    assert out.returncode == 0, out.stdout[-2000:] + out.stderr[-4000:]
    assert f"checked {len(files)} layouts" in out.stdout
