"""Host-side bounds checks of kernel launches (CPU): a small driver linked
against the library's kernel objects calls the dH launch check and the dH
launcher with arguments that would write past the partials buffer, and must
see every one refused before anything is launched."""
import os
import subprocess

import pytest

from chunked_sparse_kl_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _have_tools():
    try:
        B.hipcc()
    except RuntimeError:
        return False
    return os.path.exists(os.path.join(B.BUILD_DIR, "kd_gemm.o"))


@pytest.mark.skipif(not _have_tools(), reason="needs hipcc and the kernel objects of the regular build")
def test_dh_launch_refuses_out_of_bounds_splits(tmp_path):
    hipcc = B.hipcc()
    drv_o, exe = str(tmp_path / "guard.o"), str(tmp_path / "guard")
    r = subprocess.run([hipcc, *B.compile_flags(), "-c", os.path.join(ROOT, "tests", "guard_driver.cpp"),
                        "-o", drv_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([hipcc, f"--offload-arch={B.ARCH}", drv_o, os.path.join(B.BUILD_DIR, "kd_gemm.o"),
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout, r.stderr[-2000:])
