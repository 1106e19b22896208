"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code
(no GPU needed).

* The C oracle, built by gcc with -fsanitize=address,undefined, runs the
  oracle's pin tests (tests/test_oracle.py).
* The HIP library with its host code instrumented (each -fsanitize= after
  -Xarch_host, so no device code is built with a sanitizer) runs the C-ABI
  boundary tests (tests/test_boundary.py): argument validation, sizes,
  workspace queries and error paths, all on the host.

Each suite runs in a subprocess with the matching sanitizer runtime preloaded
and stops at the first report (halt_on_error / -fno-sanitize-recover).  Leak
detection is off: the Python interpreter and the HIP runtime keep their
allocations until exit by design.
"""
import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_quantized_matmul_fp32_amd", "csrc")
ORACLE_SRC = os.path.join(ROOT, "oracle", "vq_oracle.c")
HIPCC = "/opt/rocm/bin/hipcc"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run_suite(preload, setup, tests):
    code = ("import sys; sys.path.insert(0, %r)\n%s\nimport pytest\n"
            "sys.exit(pytest.main(['-x', '-q', '-p', 'no:cacheprovider'] + %r))\n" % (ROOT, setup, tests))
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc missing")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call([gcc, "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                           "-fPIC", "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", "-o", lib, ORACLE_SRC, "-lm"])
    rt = [subprocess.check_output([gcc, "-print-file-name=" + n], text=True).strip()
          for n in ("libasan.so", "libubsan.so")]
    setup = ("import os, oracle\noracle._LIB_PATH = %r\nos.utime(oracle._LIB_PATH)\n"
             "assert oracle.lib()._name == %r\n" % (lib, lib))
    out = _run_suite(" ".join(rt), setup, ["tests/test_oracle.py"])
    assert " passed" in out


def _asan_runtime():
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return cands[-1] if cands else None


def test_host_api_under_asan_ubsan(tmp_path):
    rt = _asan_runtime()
    if not os.path.exists(HIPCC) or rt is None:
        pytest.skip("hipcc or the clang ASan runtime missing")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + san

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC] + flags + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libvq_san.so")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + san[:4] + ["-o", lib] + objs)
    nm = subprocess.run(["nm", "-u", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm, "host code not instrumented"
    setup = ("import block_quantized_matmul_fp32_amd as vq\nvq.LIB_PATH = %r\n"
             "assert vq.lib()._name == %r\n" % (lib, lib))
    out = _run_suite(rt, setup, ["tests/test_boundary.py"])
    assert " passed" in out
