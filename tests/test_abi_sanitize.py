"""The C ABI's argument validation under host AddressSanitizer and
UndefinedBehaviorSanitizer.  `api.hip` (validation, size arithmetic,
workspace layout) is rebuilt with the sanitizers on its host code only and
linked with the library's other objects and a C++ driver
(`tests/csrc/abi_sanitize.cpp`) that calls every entry point with extreme
sizes, bad blocks and budgets, NULL and misaligned pointers; each call is a
host query or is rejected before any device work, so no GPU is needed.  Any
signed overflow, bad shift or out-of-bounds access in that host code aborts
the driver."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "dense_sparse_w4a4_amd")
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and shutil.which("g++")), reason="needs hipcc and g++")
def test_abi_validation_under_host_sanitizers(tmp_path):
    from dense_sparse_w4a4_amd import build
    objdir = os.path.join(PKG, "_build")
    others = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in build.sources()
              if not s.endswith("api.hip")]
    if not all(os.path.exists(o) for o in others):
        build.build(verbose=False)
    api_o = tmp_path / "api_sanitized.o"
    # sanitizers on the host pass only (each -fsanitize behind -Xarch_host)
    subprocess.run([HIPCC, *build.FLAGS, "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                    "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", str(api_o)],
                   check=True, capture_output=True)
    exe = tmp_path / "abi_sanitize"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    f"-I{os.path.join(ROOT, 'include')}", os.path.join(HERE, "csrc", "abi_sanitize.cpp"),
                    str(api_o), *others, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                    "-o", str(exe)], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert out.returncode == 0, out.stdout[-3000:] + out.stderr[-3000:]
    assert "failures 0" in out.stdout
