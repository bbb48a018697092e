"""CPU sanitizer builds (AddressSanitizer + UndefinedBehaviorSanitizer, no recovery):
  - the oracle (oracle/rl_oracle.c, gcc) driven through every entry point and error path by
    tests/host/oracle_san.c;
  - the host code of the HIP library (hipcc: sanitizers on the host side only) driven by
    tests/host/abi_san.cpp through the C ABI's argument validation, workspace sizing, error
    strings and the expert cache's planning mode -- the paths that run before any launch, so no
    GPU is needed.
Each exercise exits 0 only if every call returned what its header documents; a sanitizer
finding aborts it with a report on stderr."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN_REPORT = ("AddressSanitizer", "runtime error", "UndefinedBehaviorSanitizer", "LeakSanitizer")


def _run(exe, env_extra):
    env = dict(os.environ, **env_extra)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert not any(s in r.stderr for s in SAN_REPORT), r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-pthread", os.path.join(ROOT, "oracle", "rl_oracle.c"),
                    os.path.join(HERE, "host", "oracle_san.c"), "-lm", "-o", exe], check=True)
    out = _run(exe, {"ASAN_OPTIONS": "detect_leaks=1"})
    assert "all checks passed" in out


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not available")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc"
    # sanitizers apply to the host side only (each -fsanitize preceded by -Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "routed_experts_bit_amd", "csrc")]
    objs = []
    for src in ("rl_moe.hip", "rl_cache.hip"):
        o = str(tmp_path / (src + ".o"))
        subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *san, "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops", *inc, "-c",
                        os.path.join(ROOT, "routed_experts_bit_amd", "csrc", src), "-o", o],
                       check=True, capture_output=True)
        objs.append(o)
    drv = str(tmp_path / "abi_san.o")
    subprocess.run([hipcc, "-O1", "-g", "-std=c++17", *san, *inc, "-c", os.path.join(HERE, "host", "abi_san.cpp"),
                    "-o", drv], check=True, capture_output=True)
    exe = str(tmp_path / "abi_san")
    subprocess.run([hipcc, *san, drv, *objs, "-o", exe], check=True, capture_output=True)
    # the HIP runtime's own allocations outlive main: leak checking is for the oracle only
    out = _run(exe, {"ASAN_OPTIONS": "detect_leaks=0"})
    assert "all checks passed" in out
