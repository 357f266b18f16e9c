"""Builds libfkv.so (all HIP sources under csrc/) for gfx950 with hipcc, in-tree, and the
probe library (csrc/probe/, libfkv_probe.so: not part of the library): the benchmark's
stream-read probe and the check of the E4M3 conversion helper run by the GPU tests."""

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libfkv.so")
PROBE_SRCS = [os.path.join(CSRC, "probe", f) for f in ("stream_read.hip", "e4m3_check.hip")]
PROBE_OUT = os.path.join(HERE, "libfkv_probe.so")
OBJ_DIR = os.path.join(HERE, "_build")
SOURCES = ["fkv_api.hip", "fkv_insert.hip", "fkv_decode.hip", "fkv_rows.hip", "fkv_m32.hip", "fkv_noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
    # no packed fp32 instructions anywhere (the compiler would otherwise form them from float code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division for the quantiser
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # builtin MFMAs in VGPR form (their results feed VALU code); accumulators that must live
    # in AGPRs are pinned there by inline asm
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # the path produces no NaN (masks are bit operations, stale V is zeroed): max needs no NaN quieting
    "-fno-honor-nans",
]


def _compile(src):
    obj = os.path.join(OBJ_DIR, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in (r.stderr or "").splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def build(verbose=False):
    """Compile every source and link libfkv.so. Always recompiles."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES) + len(PROBE_SRCS)) as ex:
        results = list(ex.map(_compile, SOURCES + PROBE_SRCS))
    probe_objs = [o for o, _ in results[len(SOURCES):]]
    results = results[:len(SOURCES)]
    objs = [o for o, _ in results]
    if verbose:
        for (_, err), src in zip(results, SOURCES):
            if err.strip():
                print(f"[{src}]\n{err}", file=sys.stderr)
    tmp = OUT + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", PROBE_OUT + ".tmp"] + probe_objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe link failed:\n{r.stderr}")
    os.replace(PROBE_OUT + ".tmp", PROBE_OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
