"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the host code, on the CPU.

* The C oracle (oracle/idx_oracle.c) built by gcc with -fsanitize=address,undefined
  runs the oracle pins (tests/test_oracle_pins.py).
* The library's host code (argument checks, workspace sizing, launch setup in
  two_level_top_amd/csrc/*.hip) built by hipcc with the sanitizers on the host
  side only (-Xarch_host before each -fsanitize=; the gfx950 code is built as
  usual) runs the host-side ABI and binding tests, which call every entry
  point with bad arguments and never launch a kernel.

Each run is a child pytest process with the matching sanitizer runtime
preloaded (the Python interpreter itself is not instrumented); a sanitizer
report fails the child.  The builds are cached under _build/sanitize/ by a
hash of their sources and flags.
"""

from __future__ import annotations

import glob
import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CACHE = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ORACLE_FLAGS = ["-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11",
                "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                "-fno-omit-frame-pointer"]
HIP_FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]
HIP_LINK = ["--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _digest(files, flags):
    h = hashlib.sha256(" ".join(flags).encode())
    for f in sorted(files):
        h.update(f.encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}")


def _child_pytest(tests, env_extra, preload):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *tests], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for marker in ("ERROR: AddressSanitizer", "runtime error:"):
        assert marker not in out, out[-4000:]
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_pins_under_asan_ubsan():
    src = os.path.join(ROOT, "oracle", "idx_oracle.c")
    lib = os.path.join(CACHE, f"liboracle_{_digest([src], ORACLE_FLAGS)}.so")
    if not os.path.exists(lib):
        os.makedirs(CACHE, exist_ok=True)
        _run(["gcc", *ORACLE_FLAGS, "-o", lib + ".tmp", src, "-lm"])
        os.replace(lib + ".tmp", lib)
    preload = ":".join(subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True,
                                      text=True).stdout.strip() for n in ("libasan.so", "libubsan.so"))
    out = _child_pytest(["tests/test_oracle_pins.py"], {"IDX_ORACLE_LIBRARY": lib}, preload)
    assert " passed" in out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_library_host_code_under_asan_ubsan():
    csrc = os.path.join(ROOT, "two_level_top_amd", "csrc")
    srcs = sorted(glob.glob(os.path.join(csrc, "*.hip")))
    deps = srcs + sorted(glob.glob(os.path.join(csrc, "*.h"))) + [os.path.join(ROOT, "include", "idx.h")]
    tag = _digest(deps, HIP_FLAGS + HIP_LINK)
    lib = os.path.join(CACHE, f"libidx_{tag}.so")
    if not os.path.exists(lib):
        objdir = os.path.join(CACHE, f"obj_{tag}")
        os.makedirs(objdir, exist_ok=True)
        inc = ["-I", os.path.join(ROOT, "include"), "-I", csrc]
        objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
        with ThreadPoolExecutor(min(8, len(srcs))) as ex:
            list(ex.map(lambda so: _run([HIPCC, *HIP_FLAGS, *inc, "-c", so[0], "-o", so[1]]),
                        zip(srcs, objs)))
        _run([HIPCC, *HIP_LINK, "-o", lib + ".tmp", *objs])
        os.replace(lib + ".tmp", lib)
        shutil.rmtree(objdir, ignore_errors=True)
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("clang ASan runtime not found")
    out = _child_pytest(["tests/test_abi_host.py", "tests/test_binding_host.py"],
                        {"IDX_LIBRARY": lib}, rt[0])
    assert " passed" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_the_preloaded_runtime_reports_a_planted_overflow(tmp_path):
    """The harness itself: a one-past-the-end heap read, built and preloaded the
    same way, must be reported (otherwise a clean run above would prove nothing)."""
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\n"
                   "int planted(int n) { int* p = malloc(n * sizeof(int)); int v = p[n]; free(p); return v; }\n")
    lib = str(tmp_path / "libplanted.so")
    _run(["gcc", *ORACLE_FLAGS, "-o", lib, str(src)])
    preload = ":".join(subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True,
                                      text=True).stdout.strip() for n in ("libasan.so", "libubsan.so"))
    env = dict(os.environ)
    env.update(SAN_ENV)
    env["LD_PRELOAD"] = preload
    r = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({lib!r}).planted(4)"],
                       env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
