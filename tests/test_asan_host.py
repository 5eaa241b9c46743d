"""CPU: the C ABI's host-side validation under the address and
undefined-behaviour sanitizers.

api.hip (the entry points' argument checks, dispatch and size arithmetic) is
compiled with both sanitizers on its host side only and linked with the
library's other objects as built.  Two drivers then run against that build,
neither of which reaches the GPU:

* tests/asan/abi_host_checks.cpp calls every entry point with rejected
  arguments, documented no-ops and sizes at their limits;
* tests/test_abi.py's CPU tests run through the Python binding, with the
  sanitizer runtime preloaded and LORA_MI355X_LIB pointing at the build.

Undefined behaviour aborts (no recovery), so any report fails the test."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gemm_lora_shrink_amd")
HERE = os.path.dirname(os.path.abspath(__file__))
OBJECTS = ("segments", "shrink", "bgmv", "sgmv", "fused", "embedding", "slots", "mask")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc is not available")


def _rocm():
    return os.path.dirname(os.path.dirname(os.path.realpath(shutil.which("hipcc"))))


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd[:3])} ... failed:\n{res.stdout[-3000:]}\n{res.stderr[-3000:]}"
    return res


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    rt = subprocess.run(["hipcc", "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    if not rt or not os.path.exists(rt):
        pytest.skip("the sanitizer runtime is not installed")
    objs = [os.path.join(PKG, "_build", f"{n}.o") for n in OBJECTS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library has not been built")
    d = tmp_path_factory.mktemp("asan")
    api_o, lib = str(d / "api_san.o"), str(d / "liblora_san.so")
    _run(["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN, "-I", os.path.join(ROOT, "include"),
          "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", api_o])
    _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-o", lib, api_o, *objs])
    return d, lib, rt


def test_c_driver_under_sanitizers(sanitized):
    d, lib, _ = sanitized
    exe = str(d / "abi_host_checks")
    rocm = _rocm()
    # a plain C++ program (clang++, no device code), linked against the build
    _run([os.path.join(rocm, "llvm", "bin", "clang++"), "-D__HIP_PLATFORM_AMD__", "-O1", "-g",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
          os.path.join(HERE, "asan", "abi_host_checks.cpp"), lib, "-o", exe,
          f"-Wl,-rpath,{d}", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"])
    res = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"), timeout=120)
    assert "host checks passed" in res.stdout
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr


def test_binding_checks_under_sanitizers(sanitized):
    _, lib, rt = sanitized
    env = dict(os.environ, LD_PRELOAD=rt, LORA_MI355X_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:detect_odr_violation=0")
    probe = _run([sys.executable, "-c", "import gemm_lora_shrink_amd as g; g._load(); "
                  "print(sum('liblora_san' in l for l in open('/proc/self/maps')))"], env=env, cwd=ROOT, timeout=300)
    assert int(probe.stdout.split()[-1]) > 0, "the sanitized build was not the one loaded"
    res = _run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi.py"), "-q", "-x", "-m", "not gpu",
                "-p", "no:cacheprovider"], env=env, cwd=ROOT, timeout=600)
    assert " passed" in res.stdout
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr + res.stdout
