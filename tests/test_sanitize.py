"""Host-side sanitizer pass (CPU only): the oracle built with gcc's
AddressSanitizer and UndefinedBehaviorSanitizer runs its pin tests, and the
library's host code (argument checks, plan, workspace carving, the C ABI) built
with clang's AddressSanitizer and UndefinedBehaviorSanitizer (host pass only; the
device code is unchanged) runs the C-ABI tests. Each run is a subprocess with the
sanitizer runtime preloaded; any report fails the run."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.slow


def _env(extra):
    env = dict(os.environ)
    env.update(extra)
    env["OMP_NUM_THREADS"] = "2"
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    return env


def _run_pytest(files, env):
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m",
           "not gpu and not slow", *files]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_oracle_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_asan.so")
    src = os.path.join(ROOT, "oracle", "moba_oracle.c")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
                    "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-o", lib, src, "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True,
                           text=True, check=True).stdout.strip()
    env = _env({"MOBA_ORACLE_LIB": lib, "LD_PRELOAD": asan + " " + ubsan,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    _run_pytest(["tests/test_oracle_pins.py", "tests/test_oracle_backward_pins.py"], env)


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    from block_sparse_attention_causal_amd import build as hip_build
    flags = [f for f in hip_build.FLAGS if f != "-O3"] + [
        "-O1", "-g", "-fno-omit-frame-pointer",
        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    objs = []
    for src in sorted(glob.glob(os.path.join(ROOT, "block_sparse_attention_causal_amd", "csrc",
                                             "*.hip"))):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run([hip_build.HIPCC, *flags, "-c", src, "-o", obj], check=True,
                       capture_output=True)
        objs.append(obj)
    lib = str(tmp_path / "libmoba_asan.so")
    subprocess.run([hip_build.HIPCC, "-shared", "-fPIC", "--offload-arch=" + hip_build.ARCH,
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-o", lib, *objs], check=True, capture_output=True)
    env = _env({"MOBA_LIB": lib, "LD_PRELOAD": rt[-1],
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    _run_pytest(["tests/test_abi.py"], env)
