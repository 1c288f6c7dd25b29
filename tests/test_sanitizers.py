"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle (``oracle/wkv7_oracle.c``) on small ragged shapes: every
  entry point, with its decode = forward and chunked = sequential identities.
* The C ABI layer (``wkv7_api.cpp``, host code only; the kernel launchers are
  stubs that report a launch error): every validation path and size query,
  including descriptors near the integer limits, where an overflow in size
  arithmetic would show as undefined behaviour.

Both are built with gcc/g++ and ``-fsanitize=address,undefined
-fno-sanitize-recover=all``, so any report fails the run.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr[-4000:]}"
    return res


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", *SAN, "-fopenmp", "-o", exe, os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "wkv7_oracle.c"), "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="1")
    out = _run([exe], env=env).stdout
    assert "0 failed checks" in out


@pytest.mark.skipif(not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"), reason="no HIP headers")
def test_abi_validation_under_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "rwkv_wkv7_delta_amd", "csrc"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    objs = []
    for src in (os.path.join(ROOT, "rwkv_wkv7_delta_amd", "csrc", "wkv7_api.cpp"),
                os.path.join(HERE, "launch_stubs.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run(["g++", "-std=c++17", *SAN, *inc, "-c", src, "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "abi_driver.o")
    _run(["gcc", "-std=c11", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(HERE, "abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run(["g++", *SAN, "-o", exe, drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    # The HIP runtime keeps allocations until exit (device queries): leaks are
    # not checked here, memory errors and undefined behaviour are.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    out = _run([exe], env=env).stdout
    assert "0 failed checks" in out
