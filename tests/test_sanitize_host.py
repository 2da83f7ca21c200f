"""The oracle (oracle/hy_oracle.c) and the host input generator (hy_inputs/gen_host.c)
built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host code only), and
the CPU pins of both run against those builds in a child process: any out-of-bounds
access, use after free or undefined behaviour (signed overflow, bad shift, misaligned
access ...) aborts the child and fails this test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def _gcc_lib(src, out):
    subprocess.run(["gcc", *SAN, "-ffp-contract=off", "-fPIC", "-shared", "-pthread", "-Wall", src, "-o", out,
                    "-lm"], check=True, capture_output=True, text=True)


@pytest.mark.timeout(600)
def test_oracle_and_generator_pins_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan not available")
    ora = str(tmp_path / "libhy_oracle_san.so")
    gen = str(tmp_path / "libhy_gen_san.so")
    _gcc_lib(os.path.join(ROOT, "oracle", "hy_oracle.c"), ora)
    _gcc_lib(os.path.join(ROOT, "hy_inputs", "gen_host.c"), gen)
    env = dict(os.environ, LD_PRELOAD=asan, HY_ORACLE_LIB=ora, HY_GEN_LIB=gen,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = ("import oracle, hy_inputs; oracle.lib(); hy_inputs.host_lib(); import sys; "
             "maps = open('/proc/self/maps').read(); "
             "sys.exit(0 if 'libhy_oracle_san.so' in maps and 'libhy_gen_san.so' in maps "
             "and 'libasan' in maps else 3)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, "the sanitized builds were not the ones loaded:\n" + r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_oracle_pins.py", "tests/test_inputs.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=540)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
