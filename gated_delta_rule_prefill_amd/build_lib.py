"""Compile the gfx950 HIP library libgdn.so in-tree (hipcc, no JIT, no torch extension).

Every source is compiled on each call (objects in parallel), then linked into
gated_delta_rule_prefill_amd/libgdn.so. libgdn_debug.so is the same library with the
C-ABI layer built with GDN_DEBUG_CHECKS (host-side checks that read device arguments, such
as distinct slot indices, and therefore synchronise the stream); the kernels are shared.
"""
import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build", "gdn")
LIB = os.path.join(HERE, "libgdn.so")
LIB_DEBUG = os.path.join(HERE, "libgdn_debug.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["gdn_api.cpp", "decode.hip", "conv1d.hip", "prefill.hip", "prefill_bf16.hip",
           "prefill_f32.hip", "prefill_conv_bf16.hip", "prefill_conv_f32.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"),
          "-I", CSRC]
DEVICE = ["-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-munsafe-fp-atomics"]


def _compile(src: str, verbose: bool, defines=(), tag: str = "") -> str:
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    cmd = ([HIPCC] + COMMON + DEVICE + ["-D" + d for d in defines] +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l).strip()
    if warn and verbose:
        print(warn, flush=True)
    return obj


def _link(objs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, out)


def build(verbose: bool = False, jobs: int = 0) -> str:
    jobs = jobs or min(len(SOURCES) + 1, max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        debug_api = ex.submit(_compile, "gdn_api.cpp", verbose, ("GDN_DEBUG_CHECKS",), "_debug")
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
        dbg = debug_api.result()
    _link(objs, LIB, verbose)
    _link([dbg] + [o for o in objs if not o.endswith("gdn_api.o")], LIB_DEBUG, verbose)
    return LIB


if __name__ == "__main__":
    import time
    t = time.time()
    print(build(verbose=True), f"({time.time() - t:.1f} s)")
