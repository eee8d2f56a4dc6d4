"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer run of the C ABI.

Builds the library with its host code (argument validation, aliasing checks,
workspace planning, launch set-up) instrumented, device code unchanged, and
runs the CPU ABI tests against it in a child process that preloads the
sanitizer runtime.  No GPU is used: every call in those tests returns before
a launch.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

import pytest

from recurrent_inverse_scan_amd import build as vla_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitized")
# Each sanitizer flag applies to the host pass only.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _build_sanitized() -> str:
    cc = vla_build.hipcc()
    os.makedirs(OUT, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", vla_build.CSRC]
    flags = [f for f in vla_build.HIP_FLAGS if not f.startswith("-Rpass")] + SAN_FLAGS

    def one(src):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        subprocess.run([cc, *flags, *inc, "-c", os.path.join(vla_build.CSRC, src), "-o", obj],
                       check=True, capture_output=True, text=True)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, vla_build.SOURCES))
    lib = os.path.join(OUT, "libvla_sanitized.so")
    subprocess.run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN_FLAGS, "-o", lib, *objs],
                   check=True, capture_output=True, text=True)
    return lib


def test_abi_under_address_and_ub_sanitizers():
    rt = _runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this ROCm install")
    try:
        lib = _build_sanitized()
    except subprocess.CalledProcessError as e:
        pytest.fail(f"sanitized build failed:\n{e.stderr[-4000:]}")
    env = dict(os.environ, VLA_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    report = (res.stdout + res.stderr)[-6000:]
    assert res.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in report and "runtime error:" not in report, report
