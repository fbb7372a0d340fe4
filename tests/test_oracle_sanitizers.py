"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle source is built a second time with gcc's -fsanitize=address,undefined (every
finding fatal), and the oracle's pin suite and property tests run against that build in a
child process with the sanitizer runtimes preloaded. Out-of-bounds accesses in the packed
varlen indexing, the DeltaLog ring of log entries or the per-thread work split, and
undefined arithmetic (signed overflow in index products, bad shifts) would stop the run.
"""
import os
import subprocess
import sys

import pytest

from oracle.build import SRC

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.parametrize("suite", ["test_oracle_pins.py", "test_oracle_properties.py"])
def test_oracle_under_sanitizers(suite, tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC", "-shared", "-pthread",
                    "-Wall", "-Wextra", "-o", lib, SRC, "-lm"], check=True)
    logs = tmp_path / "reports"
    logs.mkdir()
    # reports go to files: the child's pytest captures file descriptor 2 around each test
    env = dict(os.environ, GDN_ORACLE_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=1:log_path={logs}/asan",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={logs}/ubsan")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", suite)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = "".join(open(logs / f).read() for f in sorted(os.listdir(logs)))
    assert reports == "", reports[-4000:]
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "passed" in r.stdout, out[-4000:]
