"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI.

kd_api.cpp (planning, validation, orchestration, timing records) and a small
driver (tests/asan_driver.cpp) are compiled with the sanitizers on the host
pass only (-Xarch_host before each -fsanitize=), linked with the kernel
objects of the regular build, and run on the CPU: the driver walks every
entry point along its host-only paths (no device work).  Needs hipcc and the
objects that chunked_sparse_kl_amd.build writes.
"""
import os
import shutil
import subprocess

import pytest

from chunked_sparse_kl_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_OBJS = ["kd_kernels.o", "kd_gemm.o", "kd_topk.o", "kd_compare.o"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _have_tools():
    try:
        B.hipcc()
    except RuntimeError:
        return False
    return all(os.path.exists(os.path.join(B.BUILD_DIR, o)) for o in KERNEL_OBJS)


@pytest.mark.skipif(not _have_tools(), reason="needs hipcc and the kernel objects of the regular build")
def test_abi_host_paths_under_asan_ubsan(tmp_path):
    hipcc = B.hipcc()
    flags = [f for f in B.compile_flags() if f not in ("-O3",)] + ["-O1", "-g"]
    api_o = str(tmp_path / "kd_api_san.o")
    drv_o = str(tmp_path / "driver_san.o")
    exe = str(tmp_path / "kd_host_san")
    for src, obj in ((os.path.join(B.CSRC, "kd_api.cpp"), api_o),
                     (os.path.join(ROOT, "tests", "asan_driver.cpp"), drv_o)):
        r = subprocess.run([hipcc, *flags, *SAN, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
    objs = [os.path.join(B.BUILD_DIR, o) for o in KERNEL_OBJS]
    r = subprocess.run([hipcc, f"--offload-arch={B.ARCH}", *SAN, drv_o, api_o, *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    # the HIP runtime keeps process-lifetime allocations: leak reports are not the subject here
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
