"""The quantiser's hardware conversion helper (e4m3_cvt2: two fp32 values to two E4M3FN bytes,
round to nearest even) gives the bytes of the integer encoder e4m3_encode for every fp32 bit
pattern of magnitude below 448, each value in its own byte of the packed word, and a NaN code
for every NaN; the encoder only uses the helper when every quotient of a chunk is below 448.
Runs csrc/probe/e4m3_check.hip (built into libfkv_probe.so) over all 2^32 patterns."""

import ctypes
import os

import pytest
import torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_hardware_conversion_matches_the_encoder_below_448():
    path = os.path.join(ROOT, "fp8_kv_paged_amd", "libfkv_probe.so")
    assert os.path.exists(path), "libfkv_probe.so is missing: run __graft_entry__.build()"
    lib = ctypes.CDLL(path)
    lib.fkv_probe_e4m3_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.fkv_probe_e4m3_check.restype = ctypes.c_int
    counts = torch.zeros(5, dtype=torch.int64, device="cuda")
    examples = torch.zeros(97, dtype=torch.int32, device="cuda")
    rc = lib.fkv_probe_e4m3_check(ctypes.c_void_p(counts.data_ptr()), ctypes.c_void_p(examples.data_ptr()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    below, above, inf, nan, nan_not_nan = counts.cpu().tolist()
    ex = examples.cpu().numpy().astype("uint32")
    shown = [(hex(ex[1 + 3 * i]), hex(ex[2 + 3 * i]), hex(ex[3 + 3 * i])) for i in range(min(int(ex[0]), 8))]
    assert below == 0, shown
    assert nan_not_nan == 0
    # outside the helper's range the encoder does not use it (saturation, infinities, NaN signs)
    print("patterns where the helper differs: >= 448", above, "infinite", inf, "NaN", nan)
