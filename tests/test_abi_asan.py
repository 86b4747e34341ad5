"""The C ABI's host-side validation under AddressSanitizer (CPU, opt-in:
GSQ_ASAN=1, since it compiles the whole library a second time). The library's
host code is built with -fsanitize=address (device code unchanged), linked
into a small C driver that exercises the validation paths and workspace
sizing on heap-allocated host arrays sized exactly as the header documents;
any out-of-bounds host access aborts the driver."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "post_weight_quantization_philox_amd", "csrc")
SOURCES = ["relax.hip", "gemm.hip", "gptq.hip", "block.hip", "abi.hip"]

pytestmark = pytest.mark.skipif(
    os.environ.get("GSQ_ASAN") != "1" or not os.path.exists("/opt/rocm/llvm/bin/clang"),
    reason="opt-in (GSQ_ASAN=1, about 30 s): rebuilds the library with host ASan")


def test_abi_validation_under_host_asan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang = "/opt/rocm/llvm/bin/clang"
    host_asan = ["-Xarch_host", "-fsanitize=address"]   # host code only
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", *host_asan,
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    objs = []
    for src in SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        subprocess.run([hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj], check=True,
                       capture_output=True)
        objs.append(obj)
    lib = str(tmp_path / "libgsq_asan.so")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *host_asan, *objs, "-o",
                    lib], check=True, capture_output=True)
    exe = str(tmp_path / "driver")
    # The C driver is host code only, built by ROCm's clang (whose ASan
    # runtime the library's host objects expect).
    subprocess.run([clang, "-g", "-fsanitize=address", f"-I{os.path.join(ROOT, 'include')}",
                    os.path.join(ROOT, "tests", "helpers", "abi_asan_driver.c"), "-o", exe,
                    f"-L{tmp_path}", "-lgsq_asan", f"-Wl,-rpath,{tmp_path}"], check=True,
                   capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "asan driver ok" in r.stdout
