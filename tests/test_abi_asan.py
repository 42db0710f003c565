"""Host-side argument checks of libssmscan.so under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU needed, no kernel launched).

The library is rebuilt with the sanitizers on its host code only (its device
code is compiled as usual but never launched), and tests/abi_asan/driver.cpp
calls every entry point with each kind of bad argument, checking the documented
status and that nothing out of bounds or undefined happens on the way.  Leak
detection is off: the HIP runtime keeps allocations until the process ends."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CSRC = os.path.join(ROOT, "selective_state_space_04_amd", "csrc")
SRCS = [os.path.join(CSRC, n) for n in ("ssm_scan.hip", "ssm_conv1d.hip", "ssm_gdn2.hip", "ssm_gdn2_chunk.hip")]
# the sanitizers apply to the host pass only: each -fsanitize= follows its own -Xarch_host
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def test_abi_checks_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    lib = str(tmp_path / "libssmscan_san.so")
    exe = str(tmp_path / "abi_san")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    build_lib = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", *SAN,
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *inc, *SRCS, "-o", lib]
    r = subprocess.run(build_lib, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    build_exe = [HIPCC, "-O1", "-g", "-std=c++17", *SAN, *inc, os.path.join(ROOT, "tests", "abi_asan", "driver.cpp"),
                 "-L", str(tmp_path), "-lssmscan_san", f"-Wl,-rpath,{tmp_path}", "-o", exe]
    r = subprocess.run(build_exe, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stderr[-3000:]
    assert "abi sanitizer run: ok" in run.stdout
