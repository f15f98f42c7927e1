"""AddressSanitizer over the library's host code.  The csrc/ sources are
built with ASan on the host side only (-Xarch_host; the device code is
compiled as usual and never launched) and linked with tests/asan/
abi_host_checks.c, a C driver that sends every entry point down its argument
checks, workspace planning and error paths.  No GPU is needed: the driver
makes no call that reaches a kernel."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

from hierarchical_sparse_attention_hsa_amd import build as hbuild

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "asan", "abi_host_checks.c")


def _flags():
    # the library's own flags at -O1, with ASan on the host pass only
    out = []
    for f in hbuild.CXXFLAGS:
        out.append("-O1" if f == "-O3" else f)
    return out + ["-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-g"]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_host_paths_are_clean_under_asan(tmp_path):
    hipcc = hbuild.hipcc()
    srcs = hbuild.sources()
    defines = hbuild._variant_defines(srcs)

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        r = subprocess.run([hipcc, *_flags(), *defines, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "driver.o")
    r = subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-fsanitize=address", "-I", os.path.join(
        os.path.dirname(HERE), "include"), "-c", DRIVER, "-o", drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "abi_host_checks")
    r = subprocess.run([hipcc, f"--offload-arch={hbuild.ARCH}", "-Xarch_host", "-fsanitize=address", "-o", exe,
                        *objs, drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    # leaks are not checked: the HIP runtime keeps process-lifetime allocations
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout + r.stderr)[-6000:]
