"""The library's host code under AddressSanitizer and UBSan (CPU only).

api.cpp (argument checks, workspace layouts, launch planning up to the
first HIP call) and policy.cpp (the host policy functions) are compiled
with host-side sanitizers (-Xarch_host, so no device code is instrumented)
and linked with the normally built kernel objects into tests/asan_driver.cpp,
which exercises every error path and size query that returns before device
work.  The test fails on a sanitizer report or a failed expectation.
"""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_diffusion_drafter_round_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def kernel_objects():
    objs = sorted(glob.glob(os.path.join(ROOT, "_build", "*.hip.o")))
    if not objs:
        from block_diffusion_drafter_round_amd.build import build
        build()
        objs = sorted(glob.glob(os.path.join(ROOT, "_build", "*.hip.o")))
    return objs


def test_host_code_under_asan_ubsan(kernel_objects, tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "policy.cpp"),
                os.path.join(ROOT, "tests", "asan_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", *inc, *san,
                            "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    # link objects only (a source argument would make hipcc read every input as HIP)
    exe = str(tmp_path / "asan_driver")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *san, *objs, *kernel_objects, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = run.stdout + run.stderr
    print(out[-2000:])
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert run.returncode == 0 and "OK: 0 failed" in out, out[-4000:]
