"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU:

- the oracle (oracle.c), built by gcc with both sanitizers, runs its pin suite;
- the library's host code (argument checks, planning, launch set-up), built by hipcc with
  the sanitizers on the host side only (device code is built as usual), runs the ABI tests,
  which exercise every entry point's validation without a GPU.

Each run is a subprocess with the sanitizer runtime preloaded; a finding aborts it.  A
planted out-of-bounds read checks that the sanitizers are live."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_quantized_matrix_amd", "csrc")


def _gcc_rt(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()


def _run(env_extra, args, timeout=900):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", **env_extra)
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


@pytest.fixture(scope="module")
def oracle_san(tmp_path_factory):
    d = tmp_path_factory.mktemp("oracle_san")
    so = str(d / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-o", so, os.path.join(ROOT, "oracle", "oracle.c"),
                    "-lm"], check=True)
    return so


def test_oracle_pins_under_sanitizers(oracle_san):
    pre = f"{_gcc_rt('libasan.so')} {_gcc_rt('libubsan.so')}"
    r = _run({"LD_PRELOAD": pre, "BQM_ORACLE_LIB": oracle_san},
             ["-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "tests/test_oracle_pins.py"])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


def test_sanitizer_is_live(oracle_san):
    pre = f"{_gcc_rt('libasan.so')} {_gcc_rt('libubsan.so')}"
    probe = ("import numpy as np, oracle; lib = oracle._load(); "
             "W = np.zeros(35, np.uint8); X = np.ones(64, np.float32); Y = np.zeros(1); S = np.zeros(1); "
             "lib.oracle_qmv(2, W.ctypes.data, X.ctypes.data, 1, 1, 64, Y.ctypes.data, S.ctypes.data)")
    r = _run({"LD_PRELOAD": pre, "BQM_ORACLE_LIB": oracle_san}, ["-c", probe], timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_library_host_code_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not os.path.exists(hipcc) or not rts:
        pytest.skip("hipcc or its sanitizer runtime is not installed")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-shared-libsan"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=off",
             "-fhip-fp32-correctly-rounded-divide-sqrt", "-mllvm", "-amdgpu-mfma-vgpr-form=1", *san]
    procs, objs = [], []
    for src in ("api", "repack", "qmv", "qmv_mma", "qmm"):
        obj = str(tmp_path / f"{src}.o")
        objs.append(obj)
        procs.append(subprocess.Popen([hipcc, *flags, "-c", os.path.join(CSRC, f"{src}.hip"), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE))
    for p in procs:
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, err.decode()[-2000:]
    so = str(tmp_path / "libbqm_san.so")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *san, "-o", so, *objs], check=True)
    r = _run({"LD_PRELOAD": rts[0], "BQM_LIB": so},
             ["-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
