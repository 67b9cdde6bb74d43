"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer:

- oracle/oracle.c with a driver that runs every oracle routine on seeded
  random block bytes (tests/sanitize/oracle_driver.c);
- the host side of the C ABI's argument checks (qg_api.hip, with host-only
  stand-ins for the kernel launchers) with a driver that calls the entry
  points with invalid and valid arguments and checks the documented statuses
  (tests/sanitize/api_driver.c).  No kernel is built or run.

Either build is skipped when its toolchain is missing."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-ffp-contract=off", "-o", exe, os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    r = _run([exe], env=dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert "clean" in r.stdout


@pytest.mark.skipif(not (os.path.exists(f"{ROCM}/bin/hipcc") and os.path.exists(f"{ROCM}/llvm/bin/clang++")
                         and os.path.exists(f"{ROCM}/lib/libamdhip64.so")), reason="ROCm toolchain missing")
def test_api_checks_under_asan_ubsan(tmp_path):
    csrc = os.path.join(ROOT, "gemm_gguf_block_amd", "csrc")
    # host-only objects: the sanitizer flags reach the host compiler alone
    host = [f"{ROCM}/bin/hipcc", "-x", "hip", "--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g", "-std=c++17",
            "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
    objs = []
    for src in (os.path.join(csrc, "qg_api.hip"), os.path.join(SAN, "launch_stubs.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run(host + ["-c", src, "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "api_driver.o")
    _run([f"{ROCM}/llvm/bin/clang", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          f"-I{ROCM}/include", "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(SAN, "api_driver.c"), "-o", drv])
    exe = str(tmp_path / "api_san")
    _run([f"{ROCM}/llvm/bin/clang++", "-fsanitize=address,undefined", "-o", exe, drv, *objs, f"-L{ROCM}/lib",
          "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    # HIP_VISIBLE_DEVICES empties the device list where a GPU is present, so
    # every valid call ends in QG_ERR_NO_DEVICE as the driver expects
    r = _run([exe], env=dict(SAN_ENV, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1"))
    assert "as documented" in r.stdout
