"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

`oracle_sanitize_main.c` drives every exported oracle function over small,
ragged layers (T = 0 and 1, k = 1 and k = E, experts with no token, H not a
multiple of 64, all three weight formats, quantizer edge blocks).  It is built
twice with gcc from `oracle/moe_oracle.c`: once with the oracle's own flags and
once with the sanitizers added, aborting on the first report.  The sanitized
run must finish cleanly (this includes the leak check at exit) and print the
same output digests as the plain build, so the instrumentation neither finds a
fault nor changes a result.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
MAIN_C = os.path.join(HERE, "oracle_sanitize_main.c")
ORACLE = os.path.join(ROOT, "oracle", "moe_oracle.c")
BASE_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math"]
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _build(out, extra):
    subprocess.check_call(["gcc", *BASE_FLAGS, *extra, "-o", out, MAIN_C, ORACLE, "-lm"])


def _run(exe, env_extra):
    env = dict(os.environ, OMP_NUM_THREADS="3", **env_extra)
    return subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_clean_under_asan_ubsan(tmp_path):
    plain, san = str(tmp_path / "plain"), str(tmp_path / "san")
    _build(plain, [])
    try:
        _build(san, SAN_FLAGS)
    except subprocess.CalledProcessError:
        pytest.skip("gcc cannot link the sanitizer runtimes here")
    p = _run(plain, {})
    assert p.returncode == 0, p.stderr
    s = _run(san, {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:exitcode=23",
                   "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    assert s.returncode == 0, s.stderr[-4000:]
    assert "runtime error" not in s.stderr and "Sanitizer" not in s.stderr, s.stderr[-4000:]
    lines_p, lines_s = p.stdout.splitlines(), s.stdout.splitlines()
    # 6 layer cases x 13 stages, then 3 formats x 2 and the conversions line
    assert len(lines_p) == 6 * 13 + 7
    assert lines_s == lines_p
