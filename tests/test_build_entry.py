"""The build entry point works from a tree that holds no built library, and the
package refuses loudly (ImportError at the first call) when the library is absent."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_missing_library_fails_at_first_call(tmp_path):
    code = ("import block_sparse_masked_metadata_amd as bsm\n"
            "try:\n    bsm._capi.bsm_version()\nexcept ImportError as e:\n    print('refused', e)\n"
            "else:\n    raise SystemExit('library call succeeded without a library')\n")
    env = dict(os.environ, BSM_LIB=str(tmp_path / "absent" / "libbsm.so"))
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert "refused" in out.stdout and "not built" in out.stdout


@pytest.mark.slow
def test_build_from_clean_tree(tmp_path):
    """Copy the tracked files only (no libbsm.so, no build folder) and run build()."""
    try:
        files = subprocess.run(["git", "ls-files"], cwd=ROOT, capture_output=True, text=True,
                               check=True).stdout.split()
    except (OSError, subprocess.CalledProcessError):
        pytest.skip("not a git checkout")
    for f in files:
        src = os.path.join(ROOT, f)
        if not os.path.isfile(src):
            continue
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy2(src, dst)
    pkg = tmp_path / "block_sparse_masked_metadata_amd"
    assert not (pkg / "libbsm.so").exists()
    code = ("import __graft_entry__ as g\ng.build()\n"
            "import block_sparse_masked_metadata_amd as bsm\n"
            "assert os.path.dirname(bsm.LIB_PATH) == os.path.join(os.getcwd(), "
            "'block_sparse_masked_metadata_amd')\nprint('version', bsm._capi.bsm_version())\n")
    env = {k: v for k, v in os.environ.items() if k != "BSM_LIB"}
    out = subprocess.run([sys.executable, "-c", "import os\n" + code], cwd=tmp_path, env=env,
                         capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert (pkg / "libbsm.so").exists() and "version" in out.stdout
    out = subprocess.run([sys.executable, "-m", "block_sparse_masked_metadata_amd.build"],
                         cwd=tmp_path, env=env, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
