"""The C-ABI layer's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

gdn_api.cpp (argument validation, workspace sizing and carving, status strings, the
allocation-free entry point's bookkeeping) is compiled a second time with both sanitizers on
its host code only (-Xarch_host before every sanitizer flag, so no GPU code is instrumented),
in its release and its debug form, and linked with the library's unchanged kernel objects
into a libgdn.so / libgdn_debug.so pair in a scratch folder. tests/test_abi_host.py then runs
against that pair (GDN_LIB) in a child process with the ASan runtime preloaded: an
out-of-bounds access or use after free in the validation paths, or undefined arithmetic
(signed overflow in a size product, a bad shift), stops the run.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from gated_delta_rule_prefill_amd import build_lib  # noqa: E402

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-shared-libasan"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_host_checks_under_sanitizers(tmp_path):
    asan = _asan_runtime()
    if asan is None or not os.path.exists(build_lib.HIPCC):
        pytest.skip("hipcc or the clang ASan runtime is not installed")
    kernels = [os.path.join(build_lib.BUILD, os.path.splitext(s)[0] + ".o")
               for s in build_lib.SOURCES if s != "gdn_api.cpp"]
    if not all(os.path.exists(o) for o in kernels):
        build_lib.build()
    for name, defines in (("libgdn.so", []), ("libgdn_debug.so", ["-DGDN_DEBUG_CHECKS"])):
        obj = str(tmp_path / (name + ".api.o"))
        subprocess.run([build_lib.HIPCC, "-O1", "-g", "-fno-omit-frame-pointer"]
                       + build_lib.COMMON[1:] + build_lib.DEVICE + defines + SAN
                       + ["-c", os.path.join(build_lib.CSRC, "gdn_api.cpp"), "-o", obj],
                       check=True, capture_output=True)
        subprocess.run([build_lib.HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950"] + SAN
                       + ["-o", str(tmp_path / name), obj] + kernels,
                       check=True, capture_output=True)
    logs = tmp_path / "reports"
    logs.mkdir()
    # reports go to files: the child's pytest captures file descriptor 2 around each test
    env = dict(os.environ, GDN_LIB=str(tmp_path / "libgdn.so"), LD_PRELOAD=asan,
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=1:log_path={logs}/asan",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={logs}/ubsan")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = "".join(open(logs / f).read() for f in sorted(os.listdir(logs)))
    assert reports == "", reports[-4000:]
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "passed" in r.stdout, out[-4000:]
