"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU:
the oracle (every entry point, tests/sanitize/oracle_driver.c), the C
ABI's host side (validation, the varlen planner, split arithmetic;
tests/sanitize/host_driver.cpp, with the kernel launchers stubbed) and the
multiply-and-shift division the kernels use for tile coordinates and the
rule that picks the chained sweep (tests/sanitize/fast_div_driver.cpp).  Built with gcc / g++ on lines of their
own, no GPU code involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _run(exe, env_extra):
    env = dict(os.environ, **env_extra)
    env.pop("LD_PRELOAD", None)  # the sanitizer runtime must come first on its own
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out and "ERROR:" not in out, out[-4000:]
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", *SAN, "-fopenmp", "-Wall", "-o", exe,
                    os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle",
                                                                        "attn_oracle.c"), "-lm"],
                   check=True)
    out = _run(exe, {"ASAN_OPTIONS": "detect_leaks=1", "OMP_NUM_THREADS": "2"})
    assert "all calls returned the expected status" in out


@pytest.mark.skipif(shutil.which("g++") is None or
                    not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")),
                    reason="g++ or the HIP runtime library not available")
def test_host_abi_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_driver")
    subprocess.run(["g++", *SAN, "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__",
                    f"-I{ROCM}/include", f"-I{ROOT}/include",
                    f"-I{ROOT}/exact_attention_forward_02_amd/csrc", "-o", exe,
                    os.path.join(HERE, "host_driver.cpp"),
                    os.path.join(ROOT, "exact_attention_forward_02_amd", "csrc", "attn_api.cpp"),
                    f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"],
                   check=True)
    # the HIP runtime's own allocations outlive main; leaks are not this code's
    out = _run(exe, {"ASAN_OPTIONS": "detect_leaks=0"})
    assert "all checks passed" in out


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_fast_division_is_exact(tmp_path):
    exe = str(tmp_path / "fast_div_driver")
    subprocess.run(["g++", *SAN, "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__",
                    f"-I{ROCM}/include", f"-I{ROOT}/exact_attention_forward_02_amd/csrc",
                    "-o", exe, os.path.join(HERE, "fast_div_driver.cpp")], check=True)
    out = _run(exe, {"ASAN_OPTIONS": "detect_leaks=1"})
    assert "all quotients exact" in out
    assert "chained-sweep rule as stated" in out
