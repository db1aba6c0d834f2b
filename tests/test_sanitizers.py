"""Host AddressSanitizer + UndefinedBehaviorSanitizer builds of the oracle and of the C ABI.

The oracle (plain C) is rebuilt with gcc's sanitizers and its pin tests are run against that
build; the C ABI library is rebuilt with the sanitizers on its host code only (device code is
compiled as usual and never launched here) and the argument-check tests are run against it.
Each run happens in a child process that preloads the sanitizer runtime and fails on the
first report.  No GPU is used.
"""
import glob
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run_pytest(files, env_extra, tmp_path):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu"] + files
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    (tmp_path / "log.txt").write_text(out)
    assert "runtime error" not in out, out[-4000:]
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-4000:]
    return out


def test_oracle_pins_under_asan_ubsan(tmp_path):
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fopenmp", "-fPIC", "-shared", "-o", lib,
                    os.path.join(ROOT, "oracle", "samba_oracle.c"), "-lm"], check=True)
    out = _run_pytest(["tests/test_oracle_pins.py", "tests/test_oracle_model_pins.py",
                       "tests/test_oracle_model_wiring.py"],
                      {"LD_PRELOAD": libasan, "SAMBA_ORACLE_LIB": lib}, tmp_path)
    assert "passed" in out


def test_the_sanitized_oracle_run_catches_a_planted_overflow(tmp_path):
    """The harness above really instruments the oracle: a copy whose attention score buffer is
    one entry short (window instead of window + 1 keys) must fail with an AddressSanitizer
    report on the window pin."""
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src = open(os.path.join(ROOT, "oracle", "samba_oracle.c")).read()
    good = "malloc(sizeof(double) * (window + 1))"
    assert src.count(good) == 1
    mutant = tmp_path / "oracle_short.c"
    mutant.write_text(src.replace(good, "malloc(sizeof(double) * window)"))
    lib = str(tmp_path / "liboracle_short.so")
    subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp",
                    "-fPIC", "-shared", "-o", lib, str(mutant), "-lm"], check=True)
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update({"LD_PRELOAD": libasan, "SAMBA_ORACLE_LIB": lib})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "-k", "swa_window_brute_force"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0
    assert "AddressSanitizer: heap-buffer-overflow" in r.stdout + r.stderr


@pytest.mark.skipif(torch.cuda.device_count() > 0,
                    reason="the argument-check tests use fake device pointers; they run where no GPU is visible")
def test_c_abi_checks_under_asan_ubsan(tmp_path):
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "libsamba_scan_san.so")
    san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", f]
    cmd = ([HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-shared", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"] +
           san + ["-o", lib, os.path.join(ROOT, "selective_state_space_samba_amd", "csrc", "samba_scan.hip")])
    subprocess.run(cmd, check=True, capture_output=True)
    _run_pytest(["tests/test_abi.py", "tests/test_abi_checks.py"],
                {"LD_PRELOAD": rt[-1], "SAMBA_LIB": lib}, tmp_path)
