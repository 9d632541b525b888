"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer.

The fp64 oracle (oracle/oracle.c, with OpenMP) is driven through every entry
point on small seeded shapes and with bad arguments
(tests/sanitize/oracle_drive.c); the library's launcher (gla_api.cpp, the
host side of the C ABI) is driven through its validation paths
(tests/sanitize/abi_drive.cpp), linked with the kernels' objects as they are
built.  Only host code is instrumented (each -fsanitize= applies to the host
compilation alone); no GPU is used.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "relu_linear_attention_amd", "csrc")
BUILD = os.path.join(ROOT, "relu_linear_attention_amd", "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


def _device_count() -> int:
    try:
        import torch

        return torch.cuda.device_count()
    except Exception:
        return 0


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_drive")
    rc, log = _run(["gcc", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_drive.c"), "-lm", "-o", exe])
    assert rc == 0, log
    rc, log = _run([exe], env=dict(SAN_ENV, OMP_NUM_THREADS="4"), timeout=300)
    assert rc == 0, log
    assert "runtime error" not in log and "AddressSanitizer" not in log, log


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_launcher_validation_under_asan_ubsan(tmp_path):
    from relu_linear_attention_amd import build

    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o")
            for s in build.SOURCES if s != "gla_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api = str(tmp_path / "gla_api.o")
    drv = str(tmp_path / "abi_drive.o")
    exe = str(tmp_path / "abi_drive")
    rc, log = _run([HIPCC, f"--offload-arch={build.ARCH}", "-O1", "-g", "-std=c++17"] + san + inc +
                   ["-x", "hip", "-c", os.path.join(CSRC, "gla_api.cpp"), "-o", api])
    assert rc == 0, log
    rc, log = _run([HIPCC, "-O1", "-g", "-std=c++17"] + san + inc +
                   ["-c", os.path.join(ROOT, "tests", "sanitize", "abi_drive.cpp"), "-o", drv])
    assert rc == 0, log
    rc, log = _run([HIPCC, f"--offload-arch={build.ARCH}"] + san + [drv, api] + objs + ["-o", exe])
    assert rc == 0, log
    args = ["--no-device"] if _device_count() == 0 else []
    rc, log = _run([exe] + args, env=SAN_ENV, timeout=300)
    assert rc == 0, log
    assert "runtime error" not in log and "AddressSanitizer" not in log, log
