"""The C-ABI host layer, compiled for the CPU with AddressSanitizer and UndefinedBehaviorSanitizer
and with the kernel launchers stubbed, accepts or rejects every decode shape of q_len 1..4096 x
1..64 query heads per KV head without an out-of-bounds access, and its launch counters add up
(tests/host/counter_sweep.cpp). A planted unbounded counter index (nt - 1 for a long query
window) fails this test with "index 7 out of bounds"."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HOST = os.path.join(HERE, "host")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_counter_sweep_under_sanitizers(tmp_path):
    exe = str(tmp_path / "counter_sweep")
    sources = [os.path.join(HOST, f) for f in ("api_host.cpp", "launch_stubs.cpp", "counter_sweep.cpp")]
    flags = ["-std=c++17", "-O1", "-g", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]
    sanitizers = ["-fsanitize=address,undefined"]  # host code only: g++, no device code in these sources
    r = subprocess.run(["g++"] + flags + sanitizers + sources + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout
