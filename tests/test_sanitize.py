"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the oracle (oracle/oracle.c) on a tiny layer with edge cases, and the C ABI's
argument checks (csrc/abi.cpp linked against stub launchers, so no kernel
runs), including sizes at the ends of their types, and the ragged-K
tile-queue protocol (csrc/tile_queue.h) on host threads, under ASan/UBSan
and under ThreadSanitizer.  Built with the host
compilers (gcc / g++); no GPU code is compiled or run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _run(exe, tmp_path):
    env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, cwd=str(tmp_path), timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.check_call(["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off",
                           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_driver.c"),
                           "-lm", "-o", exe])
    assert "ok: 0 checks failed" in _run(exe, tmp_path)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")),
                    reason="needs g++ and the HIP runtime library")
def test_abi_host_checks_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
                           "-I" + os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "dropless_moe_expert_amd", "csrc", "abi.cpp"),
                           os.path.join(HERE, "abi_host_checks.cpp"), "-L" + os.path.join(ROCM, "lib"),
                           "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    assert "ok: 0 checks failed" in _run(exe, tmp_path)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
@pytest.mark.parametrize("san", [SAN, ["-g", "-O1", "-fsanitize=thread"]], ids=["asan_ubsan", "tsan"])
def test_tile_queue_epochs(tmp_path, san):
    exe = str(tmp_path / "tq_san")
    subprocess.check_call(["g++", "-std=c++17", *san, "-pthread", "-D__HIP_PLATFORM_AMD__",
                           "-I" + os.path.join(ROCM, "include"),
                           "-I" + os.path.join(ROOT, "dropless_moe_expert_amd", "csrc"),
                           os.path.join(HERE, "tile_queue_check.cpp"), "-o", exe])
    out = _run(exe, tmp_path)
    assert "ok: 0 checks failed" in out and "ThreadSanitizer" not in out, out
