"""The library's host code under AddressSanitizer (CPU only).

tv_api.cpp (every entry point's argument checks and planning) and
tv_specpv.cpp (the SpecPV buffer policy) are compiled for the host with
-fsanitize=address, linked with the already built kernel objects, and driven
by tests/host/tv_host_checks.cpp: each entry point with bad arguments must
return its error code without touching a device, and the rectifying tree is
checked against its definition over 2000 random trees with exactly sized
output arrays.  Any out-of-bounds access or use after free fails the run.
"""

import os
import subprocess

import pytest

from tree_verification_attention_tv_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
CLANG = "/opt/rocm/llvm/bin/clang++"
HOST_SOURCES = ["tv_api.cpp", "tv_specpv.cpp"]


def test_host_code_under_asan(tmp_path):
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not found")
    objs = sorted(f for f in os.listdir(B.BUILD) if f.endswith(".o")) if os.path.isdir(B.BUILD) else []
    kernels = [os.path.join(B.BUILD, f) for f in objs
               if os.path.splitext(f)[0] + ".cpp" not in HOST_SOURCES]
    if not kernels:
        pytest.skip("library objects not built (run __graft_entry__.build())")
    flags = ["-std=c++17", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
             "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{B.INCLUDE}", f"-I{B.CSRC}"]
    host_objs = []
    for src in HOST_SOURCES + [os.path.join(HERE, "host", "tv_host_checks.cpp")]:
        path = src if os.path.isabs(src) else os.path.join(B.CSRC, src)
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([CLANG] + flags + ["-c", path, "-o", obj], capture_output=True,
                           text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        host_objs.append(obj)
    exe = str(tmp_path / "tv_host_checks")
    r = subprocess.run([CLANG, "-fsanitize=address", "-o", exe] + host_objs + kernels +
                       ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "host checks passed" in r.stdout, (r.stdout + r.stderr)[-4000:]
