"""AddressSanitizer check of the library's host code, on the CPU.

The library is rebuilt with AddressSanitizer on its host code only (device
code is compiled as usual and never runs here), and `host_asan_driver.cpp`
drives every host-side path of the C ABI through it: workspace sizes, the
schedule summary and step list for many shapes and both product orders
(also from several threads at once, which exercises the per-shape plan
cache), and the argument checks that reject a call before any device access.
An out-of-bounds access or use-after-free in those paths aborts the driver
with a report; the driver also checks each documented return value.
"""
import glob
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "two_sided_gptq_amd", "csrc")
SOURCES = ["common.hip", "quantize.hip", "hessian.hip", "factor.hip"]
ROCM = "/opt/rocm"


def _tools():
    hip = os.path.join(ROCM, "bin", "hipcc")
    cxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    rt = glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                "libclang_rt.asan-x86_64.so"))
    if not (os.path.exists(hip) and os.path.exists(cxx) and rt):
        pytest.skip("hipcc, clang++ or the AddressSanitizer runtime is missing")
    return hip, cxx


def test_host_code_under_address_sanitizer(tmp_path):
    hip, cxx = _tools()
    lib = tmp_path / "libbakron_asan.so"
    # sanitizer flags apply to the host pass only
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [hip, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-fhip-fp32-correctly-rounded-divide-sqrt",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_asan,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", str(lib)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    drv = tmp_path / "driver"
    asan = ["-fsanitize=address", "-fno-omit-frame-pointer"]
    subprocess.run([cxx, "-std=c++17", "-O1", "-g", *asan, "-I", os.path.join(ROOT, "include"),
                    os.path.join(HERE, "host_asan_driver.cpp"), f"-L{tmp_path}", "-lbakron_asan",
                    f"-Wl,-rpath,{tmp_path}", f"-Wl,-rpath,{ROCM}/lib", "-pthread", "-o", str(drv)],
                   check=True, capture_output=True, timeout=300)
    # leak reports are off: the library keeps its per-shape plans for the
    # life of the process by design
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([str(drv)], capture_output=True, text=True, timeout=600, env=env)
    print(r.stdout, r.stderr[-4000:])
    assert "AddressSanitizer" not in r.stderr
    assert r.returncode == 0 and "host checks passed" in r.stdout
