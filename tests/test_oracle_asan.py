"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host only).

tests/oracle_asan/driver.c calls every entry point of oracle/ssm_oracle.c and
oracle/conv_oracle.c on small seeded shapes (ragged sizes, one token, zero tokens,
several channel blocks, every conv width, with and without the optional
arguments), each buffer allocated at exactly the size the call may touch, and
checks that stepping equals the forward bit for bit.  Built with gcc and run in a
subprocess: any out-of-bounds access, use after free, leak or undefined
arithmetic aborts it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRCS = [os.path.join(ROOT, "tests", "oracle_asan", "driver.c"),
        os.path.join(ROOT, "oracle", "ssm_oracle.c"),
        os.path.join(ROOT, "oracle", "conv_oracle.c")]


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    exe = str(tmp_path / "oracle_asan")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off", *SRCS, "-o", exe, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("the sanitizer runtime is not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stderr[-3000:]
    assert "oracle sanitizer run: ok" in run.stdout
