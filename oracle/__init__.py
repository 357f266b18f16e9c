"""CPU oracle for calibrated-FP8 paged KV insertion and paged GQA decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
anything in this package: only the tests, the smoke check of the package entry
point and the bench's CPU-baseline leg use it. It shares no code, tables or
constants with the HIP library and imports nothing from it.

The oracle is plain NumPy in float64 and follows the problem statement of the
pages "Laguna S 2.1 INT4 -- calibrated FP8 KV on Intel B70" (section Contract:
explicit E4M3 KV with per-layer calibrated scalar K/V scales, unit scales for the
draft cache layers) and "Laguna S 2.1 KV-cache precision decision" (section
"What the official checkpoint requests": static, symmetric, per-tensor FP8 KV
scales; section "BF16 versus FP8 in concrete terms": 8 KV heads x 128 and the
per-token payload).

Modules:
  e4m3       -- E4M3FN decode/encode and the scaled quantiser
  paged      -- cache sizes, the pool byte layout, insertion and gather
  attention  -- dense decode attention over the dequantised cache
  normrope   -- per-head Q/K RMSNorm and RoPE ahead of the scaled insert

Every function here is pinned by a test under tests/ against something other
than itself (library routine, printed payload figures, closed forms,
invariants, brute force); none is "parity unpinned".
"""

from . import e4m3, paged, attention, normrope  # noqa: F401
